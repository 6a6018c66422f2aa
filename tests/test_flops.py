"""Closed-form pair counts against brute-force enumeration of the mask."""
import numpy as np
import pytest

from varlen_sliding_window_amd.flops import attention_flops, count_pairs, pairs_in_segment


def brute_pairs(length, window):
    n = 0
    for i in range(length):
        for j in range(length):
            if j <= i and (window <= 0 or j > i - window):
                n += 1
    return n


@pytest.mark.parametrize("length", [0, 1, 2, 7, 8, 9, 31, 64, 100])
@pytest.mark.parametrize("window", [0, -1, 1, 2, 8, 64, 1000])
def test_pairs_closed_form(length, window):
    assert pairs_in_segment(length, window) == brute_pairs(length, window)


def test_count_pairs_and_flops():
    cu = [0, 3, 3, 10, 11]
    assert count_pairs(cu, 0) == 6 + 28 + 1
    assert count_pairs(cu, 2) == 5 + 13 + 1
    f = attention_flops(cu, 0, 8, 128)
    assert f["fwd"] == 4 * 128 * 35 * 8 and f["bwd"] == 10 * 128 * 35 * 8
    rng = np.random.default_rng(0)
    for _ in range(20):
        lens = rng.integers(0, 40, size=6)
        cu = np.concatenate([[0], np.cumsum(lens)])
        w = int(rng.integers(-1, 20))
        assert count_pairs(cu, w) == sum(brute_pairs(int(x), w) for x in lens)
