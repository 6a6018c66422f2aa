"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments with the documented codes before touching a device."""
import ctypes
import os
import re

import pytest

import varlen_sliding_window_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_varlen.h")

EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_(?:varlen|delta|kda)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIBRARY_PATH):
        pytest.skip("library not built")
    return attn.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"attn_varlen_fwd", "attn_varlen_bwd", "attn_varlen_workspace_size",
            "attn_varlen_strerror", "attn_delta_fwd", "attn_delta_bwd",
            "attn_delta_bwd_workspace_size", "attn_kda_fwd", "attn_kda_workspace_size", "attn_kda_bwd",
            "attn_kda_bwd_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_version_and_strerror(lib):
    assert lib.attn_varlen_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert len(attn.strerror(code)) > 0


def test_workspace_size(lib):
    n = attn.workspace_size(16384, 64, 8, 2, 128, 4096, 512)
    # at least D (fp32 [Hq, T]) plus both tile lists
    assert n >= 8 * 16384 * 4 + 2 * 16 * (16384 // 32 + 64)
    assert n % 256 == 0
    assert attn.workspace_size(16384, 64, 8, 2, 64, 4096, 512) == n     # head dim 64
    assert attn.workspace_size(16384, 64, 8, 2, 256, 4096, 512) == n    # head dim 256
    assert attn.workspace_size(16384, 64, 8, 2, 96, 4096, 512) == 0     # head dim 96
    assert attn.workspace_size(0, 1, 8, 2, 128, 1, 0) == 0               # T = 0
    assert attn.workspace_size(100, 1, 8, 3, 128, 100, 0) == 0           # Hq % Hkv
    assert attn.workspace_size(100, 1, 8, 2, 128, 101, 0) == 0           # max_seqlen > T
    # k of T x Hkv x D bf16 must stay under 4 GiB (32-bit row offsets)
    assert attn.workspace_size((1 << 23) - 1, 1, 16, 2, 128, 4096, 0) > 0   # 4 GiB - 512 B
    assert attn.workspace_size(1 << 23, 1, 16, 2, 128, 4096, 0) == 0         # 4 GiB
    assert attn.workspace_size(1 << 22, 1, 32, 8, 256, 4096, 0) == 0     # 16 GiB


FAKE = 1 << 20  # aligned, never dereferenced: every case below fails validation first


def call_fwd(lib, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, nseq=1, T=64, hq=8, hkv=2, d=128, ms=64, w=0,
                scale=0.088, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.attn_varlen_fwd(args["q"], args["k"], args["v"], args["cu"], args["nseq"],
                               args["T"], args["hq"], args["hkv"], args["d"], args["ms"],
                               args["w"], args["scale"], args["out"], args["lse"], args["ws"],
                               args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, EINVAL), ({"cu": None}, EINVAL), ({"out": None}, EINVAL),
    ({"lse": None}, EINVAL), ({"q": FAKE + 8}, EINVAL), ({"T": 0}, EINVAL),
    ({"nseq": 0}, EINVAL), ({"hkv": 3}, EINVAL), ({"hq": 0}, EINVAL), ({"ms": 0}, EINVAL),
    ({"ms": 65}, EINVAL), ({"scale": 0.0}, EINVAL), ({"scale": -1.0}, EINVAL),
    ({"scale": float("nan")}, EINVAL), ({"scale": float("inf")}, EINVAL),
    ({"d": 96}, EUNSUPPORTED), ({"d": 32}, EUNSUPPORTED), ({"d": 512}, EUNSUPPORTED),
    ({"d": 0}, EUNSUPPORTED), ({"hq": 2, "hkv": 4}, EINVAL), ({"hq": 6, "hkv": 4}, EINVAL),
    ({"hkv": 0}, EINVAL), ({"ws": None}, EWORKSPACE), ({"wsb": 16}, EWORKSPACE),
    ({"ws": FAKE + 16}, EWORKSPACE),
])
def test_fwd_rejects(lib, over, code):
    assert call_fwd(lib, **over) == code


@pytest.mark.parametrize("cap", [-1.0, -1e-30, float("nan"), float("inf"), float("-inf")])
def test_softcap_rejects(lib, cap):
    args = [FAKE] * 4 + [1, 64, 8, 2, 128, 64, 0, 0.088, cap, 0, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.attn_varlen_fwd_ex(*args) == EINVAL
    bargs = [FAKE] * 7 + [1, 64, 8, 2, 128, 64, 0, 0.088, cap, 0, FAKE, FAKE, FAKE, FAKE,
                          1 << 30, None]
    assert lib.attn_varlen_bwd_ex(*bargs) == EINVAL


@pytest.mark.parametrize("flags", [2, 4, 0x80000000, 3])
def test_fwd_ex_rejects_unknown_flags(lib, flags):
    args = [FAKE] * 4 + [1, 64, 8, 2, 128, 64, 0, 0.088, 0.0, flags, FAKE, FAKE, FAKE, 1 << 30,
                         None]
    assert lib.attn_varlen_fwd_ex(*args) == EINVAL


@pytest.mark.parametrize("flags", [2, 4, 0x80000000, 3])
def test_bwd_ex_rejects_unknown_flags(lib, flags):
    bargs = [FAKE] * 7 + [1, 64, 8, 2, 128, 64, 0, 0.088, 0.0, flags, FAKE, FAKE, FAKE, FAKE,
                          1 << 30, None]
    assert lib.attn_varlen_bwd_ex(*bargs) == EINVAL


def test_bwd_rejects(lib):
    f = lib.attn_varlen_bwd
    base = [FAKE] * 7 + [1, 64, 8, 2, 128, 64, 0, 0.088, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    for pos, val, code in ((4, None, EINVAL), (5, None, EINVAL), (15, None, EINVAL),
                           (17, None, EINVAL), (11, 96, EUNSUPPORTED), (12, 65, EINVAL), (19, 8, EWORKSPACE),
                           (14, 0.0, EINVAL)):
        a = list(base)
        a[pos] = val
        assert f(*a) == code, (pos, val)


@pytest.mark.parametrize("window", [0, -1, -512])
def test_band_calls_need_a_window(lib, window):
    args = [FAKE] * 4 + [1, 64, 8, 2, 128, 64, window, 0.088, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.attn_varlen_band_fwd(*args) == EINVAL
    bargs = [FAKE] * 7 + [1, 64, 8, 2, 128, 64, window, 0.088, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          None]
    assert lib.attn_varlen_band_bwd(*bargs) == EINVAL


def test_band_calls_check_like_the_plain_ones(lib):
    # a null q or an unsupported head dim fail the same way with and without the band
    args = [None] + [FAKE] * 3 + [1, 64, 8, 2, 128, 64, 16, 0.088, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.attn_varlen_band_fwd(*args) == EINVAL
    args = [FAKE] * 4 + [1, 64, 8, 2, 96, 64, 16, 0.088, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.attn_varlen_band_fwd(*args) == EUNSUPPORTED


def test_delta_rejects(lib):
    f = lib.attn_delta_fwd
    base = [FAKE] * 6 + [1, 64, 2, 128, 0.088, FAKE, FAKE, 1 << 30, None]
    assert f(*base[:9], 96, *base[10:]) == EUNSUPPORTED          # head dim
    for pos, val, code in ((0, None, EINVAL), (3, None, EINVAL), (4, FAKE + 2, EINVAL),
                           (7, 0, EINVAL), (8, 0, EINVAL), (10, 0.0, EINVAL),
                           (10, float("nan"), EINVAL), (12, None, EWORKSPACE),
                           (13, 16, EWORKSPACE)):
        args = list(base)
        args[pos] = val
        assert f(*args) == code, (pos, val)
    assert lib.attn_delta_workspace_size(64, 1, 2, 128) > 0
    assert lib.attn_delta_workspace_size(64, 1, 2, 64) == 0
    assert lib.attn_delta_workspace_size(0, 1, 2, 128) == 0


def test_delta_bwd_rejects(lib):
    f = lib.attn_delta_bwd
    base = [FAKE] * 7 + [1, 64, 2, 128, 0.088] + [FAKE] * 6 + [1 << 31, None]
    for pos, val, code in ((0, None, EINVAL), (5, None, EINVAL), (5, FAKE + 8, EINVAL),
                           (12, None, EINVAL), (15, None, EINVAL), (16, FAKE + 2, EINVAL),
                           (10, 64, EUNSUPPORTED), (11, -1.0, EINVAL), (9, 0, EINVAL),
                           (17, None, EWORKSPACE), (17, FAKE + 16, EWORKSPACE),
                           (18, 1024, EWORKSPACE)):
        args = list(base)
        args[pos] = val
        assert f(*args) == code, (pos, val)


def test_delta_bwd_workspace_size(lib):
    fwd = lib.attn_delta_workspace_size(16384, 64, 8, 128)
    bwd = lib.attn_delta_bwd_workspace_size(16384, 64, 8, 128)
    chunks = 16384 // 64 + 64
    # per (chunk, head): two fp32 128 x 128 states, a 64 x 128 dU and dW
    assert bwd - fwd == chunks * 8 * (2 * 128 * 128 + 2 * 64 * 128) * 4
    assert lib.attn_delta_bwd_workspace_size(64, 1, 2, 96) == 0
    assert lib.attn_delta_bwd_workspace_size(0, 1, 2, 128) == 0


@pytest.mark.parametrize("flags", [2, 3, 0x80000000])
def test_delta_ex_rejects_unknown_flags(lib, flags):
    fargs = [FAKE] * 6 + [1, 64, 2, 128, 0.088, flags, FAKE, FAKE, 1 << 31, None]
    assert lib.attn_delta_fwd_ex(*fargs) == EINVAL
    bargs = [FAKE] * 7 + [1, 64, 2, 128, 0.088, flags] + [FAKE] * 6 + [1 << 31, None]
    assert lib.attn_delta_bwd_ex(*bargs) == EINVAL


def test_delta_saving_forward_needs_the_backward_workspace(lib):
    fwd_n = lib.attn_delta_workspace_size(64, 1, 2, 128)
    args = [FAKE] * 6 + [1, 64, 2, 128, 0.088, 1, FAKE, FAKE, fwd_n, None]
    assert lib.attn_delta_fwd_ex(*args) == EWORKSPACE


def test_kda_rejects(lib):
    f = lib.attn_kda_fwd
    base = [FAKE] * 6 + [1, 64, 2, 128, 0.088, FAKE, FAKE, 1 << 30, None]
    for pos, val, code in ((0, None, EINVAL), (3, None, EINVAL), (3, FAKE + 4, EINVAL),
                           (9, 64, EUNSUPPORTED), (10, 0.0, EINVAL), (11, None, EINVAL),
                           (12, None, EWORKSPACE), (13, 16, EWORKSPACE)):
        args = list(base)
        args[pos] = val
        assert f(*args) == code, (pos, val)
    n = lib.attn_kda_workspace_size(16384, 64, 8, 128)
    # per (chunk, head) record: four 64 x 128 and one 64 x 64 fp32 matrices and 128 decays
    assert n >= (16384 // 64 + 64) * 8 * (4 * 64 * 128 + 64 * 64 + 128) * 4
    assert lib.attn_kda_workspace_size(16384, 64, 8, 64) == 0


def test_kda_bwd_rejects(lib):
    f = lib.attn_kda_bwd
    base = [FAKE] * 7 + [1, 64, 2, 128, 0.088] + [FAKE] * 6 + [1 << 31, None]
    for pos, val, code in ((3, FAKE + 4, EINVAL), (5, None, EINVAL), (15, FAKE + 4, EINVAL),
                           (16, None, EINVAL), (10, 64, EUNSUPPORTED), (17, None, EWORKSPACE),
                           (18, 1024, EWORKSPACE)):
        args = list(base)
        args[pos] = val
        assert f(*args) == code, (pos, val)
    fwd = lib.attn_kda_workspace_size(16384, 64, 8, 128)
    bwd = lib.attn_kda_bwd_workspace_size(16384, 64, 8, 128)
    units = (16384 // 64 + 64) * 8
    # one record layout for both; the backward adds two states, dU, dW and two
    # C x C pair gradients per unit
    assert bwd - fwd == units * (2 * 128 * 128 + 2 * 64 * 128 + 2 * 64 * 64) * 4
    args = [FAKE] * 6 + [1, 64, 2, 128, 0.088, 1, FAKE, FAKE,
                         lib.attn_kda_workspace_size(64, 1, 2, 128), None]
    assert lib.attn_kda_fwd_ex(*args) == EWORKSPACE      # saving needs the backward's size
    args[11] = 2
    assert lib.attn_kda_fwd_ex(*args) == EINVAL          # unknown flag


def test_static_backward_refuses_beyond_its_scratch_before_the_device(lib):
    """attn_varlen_bwd_static checks the problem against its static scratch
    (and the usual shape rules) on the host, before looking at the device."""
    cap = lib.attn_varlen_static_scratch_bytes()
    assert cap == 16 << 20
    t = 1 << 20
    assert attn.workspace_size(t, 1, 64, 8, 128, t, 0) > cap
    args = [FAKE] * 7 + [1, t, 64, 8, 128, t, 0, 0.088, FAKE, FAKE, FAKE, None]
    assert lib.attn_varlen_bwd_static(*args) == -6          # ATTN_ESCRATCH
    bad = list(args)
    bad[11] = 96                                             # head dim
    assert lib.attn_varlen_bwd_static(*bad) == EUNSUPPORTED
    bad = list(args)
    bad[10] = 3                                              # Hq % Hkv != 0
    assert lib.attn_varlen_bwd_static(*bad) == EINVAL



def test_schedule_call_checks_its_arguments_before_the_device(lib):
    """attn_varlen_schedule validates shapes, the boundaries pointer and the
    workspace on the host, before it looks for a device."""
    n = attn.workspace_size(4096, 2, 8, 2, 128, 2048, 512)
    args = [FAKE, 2, 4096, 8, 2, 128, 2048, 512, FAKE, n, None]
    bad = list(args)
    bad[0] = None                                            # no cu_seqlens
    assert lib.attn_varlen_schedule(*bad) == EINVAL
    bad = list(args)
    bad[4] = 3                                               # Hq % Hkv != 0
    assert lib.attn_varlen_schedule(*bad) == EINVAL
    bad = list(args)
    bad[5] = 96                                              # head dim
    assert lib.attn_varlen_schedule(*bad) == EUNSUPPORTED
    bad = list(args)
    bad[9] = n - 1                                           # workspace too small
    assert lib.attn_varlen_schedule(*bad) == EWORKSPACE
    bad = list(args)
    bad[8] = None
    assert lib.attn_varlen_schedule(*bad) == EWORKSPACE
