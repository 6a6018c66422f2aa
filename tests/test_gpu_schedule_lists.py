"""The tile lists the schedule kernel leaves in the workspace, read back and
checked against their definition (every call builds them on the device from
cu_seqlens):

- each segment [a, b) is cut into tiles of 32 tokens from a; every tile
  appears exactly once in each list, none is empty, and together they cover
  every token once (a duplicated tile would rewrite identical values and
  pass every output test, so this is checked here);
- no tile is fully masked: tiles never cross a segment boundary, and each
  tile's key range (forward) or query range (backward) is non-empty;
- both lists are sorted by cost, longest first (the forward list by 64-key
  blocks over the visible keys, the backward list by 32-query blocks over
  the queries that see the tile); without a window the backward list's sort
  key is the cost of the tile's chunk of 16 neighbouring tiles from the
  segment start (that of its first tile), so that runs of the list stay
  within a document;
- the header records the tile count, T, the tile capacity and the window,
  and marks the boundaries as well formed.

The workspace layout read here is the library's own (a 256-byte header,
then the forward list and the backward list of 32-byte tile records, each
padded to 256 bytes)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synthetic import CONFIGS, make_cu_seqlens, make_custom  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import device_inputs  # noqa: E402

TILE, KBLK, QBLK = 32, 64, 32
CHUNK = 16      # tiles per sort chunk without a window


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def read_lists(ws: torch.Tensor, total_tokens: int, num_seqs: int):
    raw = ws.cpu().numpy().view(np.int32)
    cap = (total_tokens + TILE - 1) // TILE + num_seqs
    fwd_off = 256
    bwd_off = fwd_off + ((cap * 32 + 255) // 256) * 256
    header = raw[:5].copy()
    fwd = raw[fwd_off // 4: fwd_off // 4 + cap * 8].reshape(cap, 8)
    bwd = raw[bwd_off // 4: bwd_off // 4 + cap * 8].reshape(cap, 8)
    return header, cap, fwd, bwd


def expected_tiles(cu: np.ndarray):
    tiles = []
    idx = 0
    for a, b in zip(cu[:-1], cu[1:]):
        for t0 in range(int(a), int(b), TILE):
            tiles.append((t0, min(t0 + TILE, int(b)), int(a), int(b), idx))
            idx += 1
    return tiles


def fwd_cost(t0, t1, a, window):
    klo = a if window <= 0 else max(a, t0 - window + 1)
    return (t1 - klo + KBLK - 1) // KBLK


def bwd_cost(t0, t1, b, window):
    qhi = b if window <= 0 else min(b, t1 - 1 + window)
    return (qhi - t0 + QBLK - 1) // QBLK


def fwd_key(x, window):
    t0, t1, a, b, _ = x
    return fwd_cost(t0, t1, a, window)


def bwd_key(x, window):
    t0, t1, a, b, _ = x
    if window > 0:
        return bwd_cost(t0, t1, b, window)
    c0 = a + ((t0 - a) // (TILE * CHUNK)) * TILE * CHUNK
    return bwd_cost(c0, min(c0 + TILE, b), b, window)


def check_lists(cu: np.ndarray, window: int, hq: int = 8, hkv: int = 2):
    cu = np.asarray(cu, dtype=np.int32)
    t = int(cu[-1])
    mb = make_custom(cu, hq, hkv, seed=5)
    q, k, v, _, cu_dev = device_inputs(mb)
    ms = max(int(np.diff(cu).max()), 1)
    ws = attn.new_workspace(t, len(cu) - 1, hq, hkv, 128, ms, window, q.device)
    ws.fill_(0x5A)   # stale bytes everywhere: the lists must be written, not inherited
    attn.fwd(q, k, v, cu_dev, ms, window, mb.cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    header, cap, fwd, bwd = read_lists(ws, t, len(cu) - 1)
    want = expected_tiles(cu)
    n = len(want)
    eff_window = 0 if window <= 0 or window >= t else window
    assert header.tolist() == [n, t, cap, eff_window, 1], header
    want_set = set(want)
    for name, lst, cost in (("forward", fwd, lambda x: fwd_key(x, eff_window)),
                            ("backward", bwd, lambda x: bwd_key(x, eff_window))):
        got = [tuple(int(v) for v in row[:5]) for row in lst[:n]]
        assert len(set(got)) == n, f"{name}: a tile appears twice"
        assert set(got) == want_set, f"{name}: tiles differ from the segments' tiles"
        assert all(x[1] > x[0] for x in got), f"{name}: empty tile"
        work = [fwd_cost(x[0], x[1], x[2], eff_window) if name == "forward"
                else bwd_cost(x[0], x[1], x[3], eff_window) for x in got]
        assert all(c >= 1 for c in work), f"{name}: a tile with nothing to do"
        costs = [cost(x) for x in got]
        assert all(c0 >= c1 for c0, c1 in zip(costs, costs[1:])), f"{name}: not longest first"
    covered = np.zeros(t, dtype=np.int32)
    for t0, t1, *_ in want:
        covered[t0:t1] += 1
    assert np.all(covered == 1)
    print(f"[case] schedule lists: {n} tiles, window {window}, {len(cu) - 1} segments", flush=True)


@pytest.mark.parametrize("name", ["ctx4096_w512", "ctx4096_global", "ctx512_w512"])
def test_lists_of_workload(name):
    cfg = CONFIGS[name]
    cu, _ = make_cu_seqlens(cfg, 0)
    check_lists(cu, cfg.window)


@pytest.mark.parametrize("window", [0, 1, 33, 512])
def test_lists_of_edge_segments(window):
    lens = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]
    cu = np.concatenate([[0, 0], np.cumsum(lens), [sum(lens)]])
    check_lists(cu, window)


def test_lists_beyond_one_pass():
    """Over 1,024 tiles (the scheduler's multi-pass path)."""
    rng = np.random.default_rng(91)
    lens = []
    while sum(lens) < 45000:
        lens.append(int(rng.integers(1, 900)))
    lens[-1] -= sum(lens) - 45000
    cu = np.concatenate([[0], np.cumsum(lens)])
    check_lists(cu, 300, hq=4, hkv=1)
