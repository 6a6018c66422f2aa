"""The gated delta-rule oracle against closed forms and finite differences,
and plausible mistakes planted in a copy of it that the pins must catch."""
import inspect
import types

import pytest

pytest.importorskip("torch")

from oracle import delta as oracle_delta  # noqa: E402

from delta_pins import DELTA_PINS  # noqa: E402

SOURCE = inspect.getsource(oracle_delta)

# (name, original text, planted mistake); the forward's lines, which the
# backward repeats in torch, are planted in both copies.
MUTATIONS = [
    ("no decay", "alpha = np.exp(g[t, h])", "alpha = 1.0"),
    ("delta term without the decay",
     "s = alpha * s + beta[t, h] * np.outer(v[t, h] - alpha * (s @ kt), kt)",
     "s = alpha * s + beta[t, h] * np.outer(v[t, h] - (s @ kt), kt)"),
    ("plain write, no delta correction",
     "s = alpha * s + beta[t, h] * np.outer(v[t, h] - alpha * (s @ kt), kt)",
     "s = alpha * s + beta[t, h] * np.outer(v[t, h], kt)"),
    ("read before the update", "                s = alpha * s + beta[t, h] * np.outer(v[t, h] - alpha * (s @ kt), kt)\n                o[t, h] = scale * (s @ q[t, h])",
     "                o[t, h] = scale * (s @ q[t, h])\n                s = alpha * s + beta[t, h] * np.outer(v[t, h] - alpha * (s @ kt), kt)"),
    ("no reset at documents", "    for a, b in _segments(cu_seqlens):\n        for h in range(h_):\n            s = np.zeros((dv, dk))\n",
     "    for a, b in [(0, t_)]:\n        for h in range(h_):\n            s = np.zeros((dv, dk))\n"),
    ("read with the key", "o[t, h] = scale * (s @ q[t, h])", "o[t, h] = scale * (s @ kt)"),
    ("transposed write", "np.outer(v[t, h] - alpha * (s @ kt), kt)", "np.outer(kt, v[t, h] - alpha * (s.T @ kt)).T"),
    ("backward without the delta correction",
     "s = alpha * s + tb[t, h] * torch.outer(tv[t, h] - alpha * (s @ kt), kt)",
     "s = alpha * s + tb[t, h] * torch.outer(tv[t, h], kt)"),
]


@pytest.mark.parametrize("pin", DELTA_PINS, ids=lambda f: f.__name__)
def test_delta_pin(pin):
    pin(oracle_delta)


@pytest.mark.parametrize("name,original,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_delta_mutation_is_caught(name, original, planted):
    assert SOURCE.count(original) == 1, f"mutation anchor not unique/found: {original!r}"
    mod = types.ModuleType("delta_mutant")
    exec(compile(SOURCE.replace(original, planted), "delta_mutant", "exec"), mod.__dict__)
    for pin in DELTA_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return
    pytest.fail(f"no pin caught the planted mistake '{name}'")
