"""The band-block oracle against the dense oracle and closed forms, and
plausible mistakes planted in a copy of it that the pins must catch."""
import inspect
import types

import pytest

from oracle import band as oracle_band

from oracle_pins import BAND_PINS

SOURCE = inspect.getsource(oracle_band)

# (name, original text, planted mistake)
MUTATIONS = [
    ("band drops the previous block", "lo, hi = max(0, (b - 1) * window), q1", "lo, hi = q0, q1"),
    ("band ignores documents", "vis = (seg[i] == seg[j]) & (seg[i] >= 0) & (j <= i)",
     "vis = (seg[i] >= 0) & (j <= i)"),
    ("band window one too wide", "& (j > i - window)", "& (j >= i - window)"),
    ("band not causal", "& (j <= i) &", "& (j <= i + 1) &"),
    ("band dk not accumulated", "dk[lo:hi, g] += scale", "dk[lo:hi, g] = scale"),
    ("band lse missing max", "lse[h, rows] = (m + np.log(z))[:, 0]", "lse[h, rows] = np.log(z)[:, 0]"),
    ("band dS drops D", "ds = p * (dp - dd)", "ds = p * dp"),
]


@pytest.mark.parametrize("pin", BAND_PINS, ids=lambda f: f.__name__)
def test_band_pin(pin):
    pin(oracle_band)


@pytest.mark.parametrize("name,original,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_band_mutation_is_caught(name, original, planted):
    assert SOURCE.count(original) == 1, f"mutation anchor not unique/found: {original!r}"
    mod = types.ModuleType("band_mutant")
    exec(compile(SOURCE.replace(original, planted), "band_mutant", "exec"), mod.__dict__)
    for pin in BAND_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return
    pytest.fail(f"no pin caught the planted mistake '{name}'")
