"""Plant plausible mistakes in a copy of the oracle (CPU only) and require that
at least one pin catches each of them."""
import importlib.util
import inspect
import types

import pytest

from oracle import attention as oracle_attention

from oracle_pins import ALL_PINS

SOURCE = inspect.getsource(oracle_attention)

# (name, original text, planted mistake)
MUTATIONS = [
    ("window W+1 keys", "m &= j > i - window", "m &= j >= i - window"),
    ("not causal", "m = j <= i", "m = j <= i + 1"),
    ("no window", "if window > 0:\n        m &=", "if window > 10**9:\n        m &="),
    ("scale missing in dq", "dq[a:b, h] = scale * (ds @ ks)", "dq[a:b, h] = ds @ ks"),
    ("scale missing in dk", "dk[a:b, g] += scale * (ds.T @ qs)", "dk[a:b, g] += ds.T @ qs"),
    ("dS drops D", "ds = p * (dp - dd) * dcap\n            dsum", "ds = p * dp * dcap\n            dsum"),
    ("dS wrong sign", "ds = p * (dp - dd) * dcap\n            dsum",
     "ds = p * (dd - dp) * dcap\n            dsum"),
    ("dk not summed over group", "dk[a:b, g] += scale", "dk[a:b, g] = scale"),
    ("dv not summed over group", "dv[a:b, g] += p.T @ dos", "dv[a:b, g] = p.T @ dos"),
    ("dv transposed P", "dv[a:b, g] += p.T @ dos", "dv[a:b, g] += p @ dos"),
    ("dk transposed dS", "scale * (ds.T @ qs)", "scale * (ds @ qs)"),
    ("dP transposed V", "dp = dos @ vs.T", "dp = (dos @ vs.T).T"),
    ("GQA head map modulo", "g = h // group\n            qs", "g = h % k.shape[1]\n            qs"),
    ("fwd GQA head map modulo", "g = h // group\n            o, l", "g = h % k.shape[1]\n            o, l"),
    ("LSE in log2", "lse = (m + np.log(z))[:, 0]", "lse = (m + np.log2(z))[:, 0]"),
    ("LSE missing max", "lse = (m + np.log(z))[:, 0]", "lse = np.log(z)[:, 0]"),
    ("scale after softmax", "s = scale * (qs @ ks.T)", "s = qs @ ks.T"),
    ("documents ignored", "return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]",
     "return [(0, int(cu[-1]))] if cu[-1] > 0 else []"),
    ("row window off by one", "lo = max(a, i - window + 1) if window > 0 else a",
     "lo = max(a, i - window) if window > 0 else a"),
    ("row dq drops D", "ds = p * (dp - p @ dp)", "ds = p * dp"),
    ("cap derivative dropped", "ds = p * (dp - dd) * dcap\n            dsum",
     "ds = p * (dp - dd)\n            dsum"),
    ("cap derivative 1 - t", "return softcap * t, 1.0 - t * t", "return softcap * t, 1.0 - t"),
    ("cap on unscaled logits", "t = np.tanh(s / softcap)\n        return softcap * t",
     "t = np.tanh(s / scale / softcap)\n        return scale * softcap * t"),
    ("cap as hard clip", "t = np.tanh(s / softcap)\n        return softcap * t",
     "t = np.clip(s / softcap, -1.0, 1.0)\n        return softcap * t"),
    ("row cap derivative dropped", "ds = p * (dp - p @ dp) * dcap", "ds = p * (dp - p @ dp)"),
    ("key window one too short", "hi = min(b - 1, j + window - 1) if window > 0 else b - 1",
     "hi = min(b - 1, j + window - 2) if window > 0 else b - 1"),
    ("key dS drops D", "ds = p * (dp - dd) * dcap\n        dk += scale", "ds = p * dp * dcap\n        dk += scale"),
    ("key sums one head only", "for h in range(g * group, (g + 1) * group):", "for h in range(g * group, g * group + 1):"),
    ("row cap ignored", "    if softcap > 0:\n        t = np.tanh(s / softcap)\n        s = softcap * t",
     "    if softcap > 1e300:\n        t = np.tanh(s / softcap)\n        s = softcap * t"),
]


def mutated_module(original, planted):
    assert SOURCE.count(original) == 1, f"mutation anchor not unique/found: {original!r}"
    src = SOURCE.replace(original, planted)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,original,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, original, planted):
    mod = mutated_module(original, planted)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as exc:
            caught.append((pin.__name__, str(exc)[:80]))
            break
    assert caught, f"no pin caught the planted mistake '{name}'"
