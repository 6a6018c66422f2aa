"""The Kimi Delta Attention oracle against Gated DeltaNet, coordinate-axis
closed forms and finite differences, and plausible mistakes planted in a
copy of it that the pins must catch."""
import inspect
import types

import pytest

pytest.importorskip("torch")

from oracle import kimi_delta as oracle_kda  # noqa: E402

from kda_pins import KDA_PINS  # noqa: E402

SOURCE = inspect.getsource(oracle_kda)

# (name, original text, planted mistake)
MUTATIONS = [
    ("one gate for all channels", "sp = s * np.exp(g[t, h])[None, :]",
     "sp = s * np.exp(g[t, h].mean())"),
    ("gate on the value axis", "sp = s * np.exp(g[t, h])[None, :]",
     "sp = s * np.exp(g[t, h])[:, None]"),
    ("decay after the write",
     "                sp = s * np.exp(g[t, h])[None, :]\n                kt = k[t, h]\n                s = sp + beta[t, h] * np.outer(v[t, h] - sp @ kt, kt)\n",
     "                sp = s\n                kt = k[t, h]\n                s = (sp + beta[t, h] * np.outer(v[t, h] - sp @ kt, kt)) * np.exp(g[t, h])[None, :]\n"),
    ("delta term from the undecayed state", "np.outer(v[t, h] - sp @ kt, kt)",
     "np.outer(v[t, h] - s @ kt, kt)"),
    ("plain write, no delta correction", "np.outer(v[t, h] - sp @ kt, kt)",
     "np.outer(v[t, h], kt)"),
    ("read before the update",
     "                s = sp + beta[t, h] * np.outer(v[t, h] - sp @ kt, kt)\n                o[t, h] = scale * (s @ q[t, h])",
     "                o[t, h] = scale * (s @ q[t, h])\n                s = sp + beta[t, h] * np.outer(v[t, h] - sp @ kt, kt)"),
    ("no reset at documents",
     "    for a, b in _segments(cu_seqlens):\n        for h in range(h_):\n            s = np.zeros((dv, dk))\n",
     "    for a, b in [(0, t_)]:\n        for h in range(h_):\n            s = np.zeros((dv, dk))\n"),
    ("backward with one gate for all channels", "sd = st * torch.exp(tg[t, h])[None, :]",
     "sd = st * torch.exp(tg[t, h].mean())"),
]


@pytest.mark.parametrize("pin", KDA_PINS, ids=lambda f: f.__name__)
def test_kda_pin(pin):
    pin(oracle_kda)


@pytest.mark.parametrize("name,original,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_kda_mutation_is_caught(name, original, planted):
    assert SOURCE.count(original) == 1, f"mutation anchor not unique/found: {original!r}"
    mod = types.ModuleType("kda_mutant")
    exec(compile(SOURCE.replace(original, planted), "kda_mutant", "exec"), mod.__dict__)
    for pin in KDA_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return
    pytest.fail(f"no pin caught the planted mistake '{name}'")
