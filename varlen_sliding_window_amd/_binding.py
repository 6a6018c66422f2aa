"""ctypes binding of libattn_varlen.so (the C ABI in include/attn_varlen.h).

Argument marshalling only: torch supplies device memory and the current
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or the device is not a
gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libattn_varlen.so")

ATTN_OK = 0
ATTN_BWD_REUSE_SCHEDULE = 1
ATTN_FWD_REUSE_SCHEDULE = 1
ATTN_DELTA_FWD_SAVE = 1
ATTN_DELTA_BWD_REUSE = 1
STATUS_NAMES = {0: "ATTN_OK", -1: "ATTN_EINVAL", -2: "ATTN_EUNSUPPORTED",
                -3: "ATTN_EWORKSPACE", -4: "ATTN_EDEVICE", -5: "ATTN_ELAUNCH",
                -6: "ATTN_ESCRATCH"}

_lib = None

# What the last call that built a schedule (or saved delta-rule state) left in
# each workspace, keyed by the workspace's device address and size: a reuse
# that does not match is refused here, before the device-side check (which
# would turn the outputs into NaN).
_WS_RECORD: dict = {}


def _ws_key(ws) -> tuple:
    return (ws.device.index, ws.data_ptr(), ws.numel())


def _effective_window(window: int, total_tokens: int) -> int:
    return 0 if window <= 0 or window >= total_tokens else int(window)


def _check_reuse(ws, want: tuple, what: str) -> None:
    have = _WS_RECORD.get(_ws_key(ws))
    if have != want:
        raise ValueError(f"{what}: the workspace holds {have}, this call needs {want}")


class KernelStats(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("min_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {strerror(status)}")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the shared library; raise if it was not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    lib.attn_varlen_workspace_size.argtypes = [i32] * 7
    lib.attn_varlen_workspace_size.restype = sz
    lib.attn_varlen_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    ctypes.c_float, vp, vp, vp, sz, vp]
    lib.attn_varlen_fwd.restype = ctypes.c_int
    lib.attn_varlen_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                    i32, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.attn_varlen_bwd.restype = ctypes.c_int
    lib.attn_varlen_schedule.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.attn_varlen_schedule.restype = ctypes.c_int
    lib.attn_varlen_fwd_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_uint32, vp, vp,
                                       vp, sz, vp]
    lib.attn_varlen_fwd_ex.restype = ctypes.c_int
    lib.attn_varlen_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       i32, i32, ctypes.c_float, ctypes.c_float, ctypes.c_uint32,
                                       vp, vp, vp, vp, sz, vp]
    lib.attn_varlen_bwd_ex.restype = ctypes.c_int
    lib.attn_varlen_band_fwd.argtypes = lib.attn_varlen_fwd.argtypes
    lib.attn_varlen_band_fwd.restype = ctypes.c_int
    lib.attn_varlen_band_bwd.argtypes = lib.attn_varlen_bwd.argtypes
    lib.attn_varlen_band_bwd.restype = ctypes.c_int
    lib.attn_delta_workspace_size.argtypes = [i32] * 4
    lib.attn_delta_workspace_size.restype = sz
    lib.attn_delta_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                                   vp, vp, sz, vp]
    lib.attn_delta_fwd.restype = ctypes.c_int
    lib.attn_delta_bwd_workspace_size.argtypes = [i32] * 4
    lib.attn_delta_bwd_workspace_size.restype = sz
    lib.attn_delta_bwd.argtypes = [vp] * 7 + [i32, i32, i32, i32, ctypes.c_float] + [vp] * 6 + [
        sz, vp]
    lib.attn_delta_bwd.restype = ctypes.c_int
    lib.attn_kda_workspace_size.argtypes = [i32] * 4
    lib.attn_kda_workspace_size.restype = sz
    lib.attn_kda_fwd.argtypes = [vp] * 6 + [i32, i32, i32, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.attn_kda_fwd.restype = ctypes.c_int
    lib.attn_kda_bwd_workspace_size.argtypes = [i32] * 4
    lib.attn_kda_bwd_workspace_size.restype = sz
    lib.attn_kda_bwd.argtypes = [vp] * 7 + [i32, i32, i32, i32, ctypes.c_float] + [vp] * 6 + [
        sz, vp]
    lib.attn_kda_bwd.restype = ctypes.c_int
    lib.attn_kda_fwd_ex.argtypes = [vp] * 6 + [i32, i32, i32, i32, ctypes.c_float,
                                               ctypes.c_uint32, vp, vp, sz, vp]
    lib.attn_kda_fwd_ex.restype = ctypes.c_int
    lib.attn_kda_bwd_ex.argtypes = [vp] * 7 + [i32, i32, i32, i32, ctypes.c_float,
                                               ctypes.c_uint32] + [vp] * 6 + [sz, vp]
    lib.attn_kda_bwd_ex.restype = ctypes.c_int
    lib.attn_delta_fwd_ex.argtypes = [vp] * 6 + [i32, i32, i32, i32, ctypes.c_float,
                                                 ctypes.c_uint32, vp, vp, sz, vp]
    lib.attn_delta_fwd_ex.restype = ctypes.c_int
    lib.attn_delta_bwd_ex.argtypes = [vp] * 7 + [i32, i32, i32, i32, ctypes.c_float,
                                                 ctypes.c_uint32] + [vp] * 6 + [sz, vp]
    lib.attn_delta_bwd_ex.restype = ctypes.c_int
    lib.attn_varlen_bwd_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           i32, i32, ctypes.c_float, vp, vp, vp, vp]
    lib.attn_varlen_bwd_static.restype = ctypes.c_int
    lib.attn_varlen_static_scratch_bytes.argtypes = []
    lib.attn_varlen_static_scratch_bytes.restype = sz
    lib.attn_varlen_strerror.argtypes = [ctypes.c_int]
    lib.attn_varlen_strerror.restype = ctypes.c_char_p
    lib.attn_varlen_version.argtypes = []
    lib.attn_varlen_version.restype = i32
    lib.attn_varlen_profile_start.argtypes = []
    lib.attn_varlen_profile_start.restype = ctypes.c_int
    lib.attn_varlen_profile_stop.argtypes = [ctypes.POINTER(KernelStats), i32]
    lib.attn_varlen_profile_stop.restype = i32
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().attn_varlen_strerror(int(status)).decode()


def workspace_size(total_tokens: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                   head_dim: int, max_seqlen: int, window: int) -> int:
    return int(load_library().attn_varlen_workspace_size(
        total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seqlen, window))


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def new_workspace(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seqlen,
                  window, device) -> torch.Tensor:
    n = workspace_size(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       max_seqlen, window)
    if n == 0:
        raise AttnError(-1, "attn_varlen_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def schedule(cu_seqlens, total_tokens: int, max_seqlen: int, window: int, workspace,
             num_q_heads: int, num_kv_heads: int, head_dim: int):
    """attn_varlen_schedule: build the tile schedule of (cu_seqlens, window)
    into `workspace` on the current stream, for later fwd/bwd calls with
    reuse_schedule=True (ordered after it by the caller when they run on
    another stream)."""
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, nseq = int(total_tokens), cu_seqlens.numel() - 1
    lib = load_library()
    st = lib.attn_varlen_schedule(_ptr(cu_seqlens), nseq, t, int(num_q_heads), int(num_kv_heads),
                                  int(head_dim), int(max_seqlen), int(window), _ptr(workspace),
                                  workspace.numel(), _stream_handle(cu_seqlens.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_schedule")
    _WS_RECORD[_ws_key(workspace)] = ("schedule", t, nseq, _effective_window(int(window), t))


def fwd(q, k, v, cu_seqlens, max_seqlen: int, window: int, scale: float | None = None,
        out=None, lse=None, workspace=None, softcap: float = 0.0, band: bool = False,
        reuse_schedule: bool = False, check_reuse: bool = True):
    """attn_varlen_fwd (attn_varlen_fwd_ex with a soft-cap or reuse_schedule,
    attn_varlen_band_fwd when band): returns (out [T,Hq,D] bf16, lse [Hq,T] fp32).

    softcap > 0 caps every logit to softcap * tanh(logit / softcap); band runs
    the band-block formulation (window >= 1, no soft-cap).  reuse_schedule:
    `workspace` already holds the tile schedule of an earlier call with the
    same cu_seqlens, window and sizes (another layer of a stack), which this
    call uses instead of building it.  check_reuse=False skips the binding's
    own record of what the workspace holds and leaves the refusal of a
    mismatched reuse to the device (NaN outputs)."""
    _check_tensor("q", q, torch.bfloat16, 3)
    _check_tensor("k", k, torch.bfloat16, 3)
    _check_tensor("v", v, torch.bfloat16, 3)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (t, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, Hkv, D] with q's T and D")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, t), dtype=torch.float32, device=q.device)
    if reuse_schedule and workspace is None:
        raise ValueError("reuse_schedule needs a workspace that holds a schedule")
    if workspace is None:
        workspace = new_workspace(t, nseq, hq, hkv, d, max_seqlen, window, q.device)
    sched = ("schedule", t, nseq, _effective_window(int(window), t))
    if reuse_schedule and check_reuse:
        _check_reuse(workspace, sched, "attn_varlen_fwd_ex(ATTN_FWD_REUSE_SCHEDULE)")
    lib = load_library()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), nseq, t, hq, hkv, d, int(max_seqlen),
            int(window), float(scale))
    tail = (_ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream_handle(q.device))
    if band:
        if softcap or reuse_schedule:
            raise ValueError("the band-block calls take no soft-cap and no flags")
        st, where = lib.attn_varlen_band_fwd(*head, *tail), "attn_varlen_band_fwd"
    elif softcap or reuse_schedule:
        flags = ATTN_FWD_REUSE_SCHEDULE if reuse_schedule else 0
        st, where = (lib.attn_varlen_fwd_ex(*head, float(softcap), flags, *tail),
                     "attn_varlen_fwd_ex")
    else:
        st, where = lib.attn_varlen_fwd(*head, *tail), "attn_varlen_fwd"
    if st != ATTN_OK:
        raise AttnError(st, where)
    _WS_RECORD[_ws_key(workspace)] = sched
    return out, lse


def bwd(q, k, v, out, lse, dout, cu_seqlens, max_seqlen: int, window: int,
        scale: float | None = None, dq=None, dk=None, dv=None, workspace=None,
        softcap: float = 0.0, reuse_schedule: bool = False, band: bool = False,
        check_reuse: bool = True):
    """attn_varlen_bwd (attn_varlen_bwd_ex with a soft-cap or reuse_schedule,
    attn_varlen_band_bwd when band): returns (dq, dk, dv), bf16, shaped like
    q, k, v.  softcap must be the forward's.  reuse_schedule: `workspace` was
    just used by the forward call of the same layer (same cu_seqlens and
    window), whose tile schedule the backward then uses instead of rebuilding
    it.  band: the band-block formulation (window >= 1, no soft-cap, always
    rebuilds its schedule)."""
    for name, t_ in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, hq, d = q.shape
    hkv = k.shape[1]
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (hq, t):
        raise ValueError("out/dout must match q and lse must be [Hq, T]")
    if k.shape != (t, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, Hkv, D] with q's T and D")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    workspace_arg_missing = workspace is None
    if workspace is None:
        workspace = new_workspace(t, nseq, hq, hkv, d, max_seqlen, window, q.device)
    lib = load_library()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(cu_seqlens), nseq,
            t, hq, hkv, d, int(max_seqlen), int(window), float(scale))
    tail = (_ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
            _stream_handle(q.device))
    if reuse_schedule and workspace_arg_missing:
        raise ValueError("reuse_schedule needs the forward call's workspace")
    sched = ("schedule", t, nseq, _effective_window(int(window), t))
    if reuse_schedule and check_reuse:
        _check_reuse(workspace, sched, "attn_varlen_bwd_ex(ATTN_BWD_REUSE_SCHEDULE)")
    if band:
        if softcap or reuse_schedule:
            raise ValueError("the band-block calls take no soft-cap and no flags")
        st, where = lib.attn_varlen_band_bwd(*head, *tail), "attn_varlen_band_bwd"
    elif softcap or reuse_schedule:
        flags = ATTN_BWD_REUSE_SCHEDULE if reuse_schedule else 0
        st, where = (lib.attn_varlen_bwd_ex(*head, float(softcap), flags, *tail),
                     "attn_varlen_bwd_ex")
    else:
        st, where = lib.attn_varlen_bwd(*head, *tail), "attn_varlen_bwd"
    if st != ATTN_OK:
        raise AttnError(st, where)
    if not reuse_schedule:
        _WS_RECORD[_ws_key(workspace)] = sched
    return dq, dk, dv


def _grad_buffers(grads, q, k, v, g, beta):
    """The delta-rule backward's outputs: the caller's (dq, dk, dv, dg, dbeta),
    checked, or new zero-filled ones."""
    if grads is None:
        return (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v),
                torch.zeros_like(g), torch.zeros_like(beta))
    dq, dk, dv, dg, dbeta = grads
    for name, x, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v), ("dg", dg, g),
                          ("dbeta", dbeta, beta)):
        _check_tensor(name, x, like.dtype, like.dim())
        if x.shape != like.shape:
            raise ValueError(f"{name} must be shaped like its input")
    return dq, dk, dv, dg, dbeta


def bwd_static(q, k, v, out, lse, dout, cu_seqlens, max_seqlen: int, window: int,
               scale: float | None = None, dq=None, dk=None, dv=None):
    """attn_varlen_bwd_static: the backward without a workspace (the library's
    static device scratch instead; nothing is allocated by the call when dq,
    dk, dv are given).  Calls that overlap in time on one GPU race."""
    for name, t_ in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, hq, d = q.shape
    hkv = k.shape[1]
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (hq, t):
        raise ValueError("out/dout must match q and lse must be [Hq, T]")
    if k.shape != (t, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, Hkv, D] with q's T and D")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = load_library().attn_varlen_bwd_static(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, t, hq, hkv, d, int(max_seqlen), int(window), float(scale),
        _ptr(dq), _ptr(dk), _ptr(dv), _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_bwd_static")
    return dq, dk, dv


def delta_workspace_size(total_tokens: int, num_seqs: int, num_heads: int, head_dim: int) -> int:
    return int(load_library().attn_delta_workspace_size(total_tokens, num_seqs, num_heads, head_dim))


def delta_fwd(q, k, v, g, beta, cu_seqlens, scale: float | None = None, out=None,
              workspace=None, save: bool = False):
    """attn_delta_fwd(_ex): gated delta-rule linear attention forward.  q, k, v
    bf16 [T, H, D]; g, beta fp32 [T, H]; returns out bf16 [T, H, D].  With
    save=True the workspace (of delta_bwd_workspace_size bytes) keeps what a
    delta_bwd(..., reuse=True) with the same inputs and workspace needs."""
    for name, t_ in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("g", g, torch.float32, 2)
    _check_tensor("beta", beta, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, h, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or g.shape != (t, h) or beta.shape != (t, h):
        raise ValueError("q, k, v must be [T, H, D] and g, beta [T, H]")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    if workspace is None:
        n = (delta_bwd_workspace_size if save else delta_workspace_size)(t, nseq, h, d)
        if n == 0:
            raise AttnError(-1, "attn_delta_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = load_library().attn_delta_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(cu_seqlens), nseq, t, h, d, float(scale),
                                          1 if save else 0, _ptr(out), _ptr(workspace),
                                          workspace.numel(), _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_delta_fwd_ex")
    _WS_RECORD[_ws_key(workspace)] = ("delta", t, nseq, h) if save else None
    return out


def kda_workspace_size(total_tokens: int, num_seqs: int, num_heads: int, head_dim: int) -> int:
    return int(load_library().attn_kda_workspace_size(total_tokens, num_seqs, num_heads, head_dim))


def kda_fwd(q, k, v, g, beta, cu_seqlens, scale: float | None = None, out=None, workspace=None,
            save: bool = False):
    """attn_kda_fwd(_ex): Kimi Delta Attention forward.  q, k, v bf16
    [T, H, D]; g fp32 [T, H, D] (per-channel log decay); beta fp32 [T, H];
    returns out bf16 [T, H, D].  save=True keeps, in a workspace of
    kda_bwd_workspace_size bytes, what kda_bwd(..., reuse=True) needs."""
    for name, t_ in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("g", g, torch.float32, 3)
    _check_tensor("beta", beta, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, h, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape or beta.shape != (t, h):
        raise ValueError("q, k, v, g must be [T, H, D] and beta [T, H]")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    if workspace is None:
        n = (kda_bwd_workspace_size if save else kda_workspace_size)(t, nseq, h, d)
        if n == 0:
            raise AttnError(-1, "attn_kda_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = load_library().attn_kda_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(cu_seqlens), nseq, t, h, d, float(scale),
                                        1 if save else 0, _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kda_fwd_ex")
    _WS_RECORD[_ws_key(workspace)] = ("kda", t, nseq, h) if save else None
    return out


def kda_bwd_workspace_size(total_tokens: int, num_seqs: int, num_heads: int,
                           head_dim: int) -> int:
    return int(load_library().attn_kda_bwd_workspace_size(total_tokens, num_seqs, num_heads,
                                                           head_dim))


def kda_bwd(q, k, v, g, beta, dout, cu_seqlens, scale: float | None = None, workspace=None,
            reuse: bool = False, check_reuse: bool = True, grads=None):
    """attn_kda_bwd(_ex): gradients of sum(dout * out) of the Kimi Delta
    forward.  Returns dq, dk, dv (bf16 [T, H, D]), dg (fp32 [T, H, D]) and
    dbeta (fp32 [T, H]), zero-filled first.  reuse=True takes the records and
    states a kda_fwd(..., save=True) with the same inputs left in `workspace`."""
    if reuse and workspace is None:
        raise ValueError("reuse needs the workspace of a saving forward")
    for name, t_ in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("g", g, torch.float32, 3)
    _check_tensor("beta", beta, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, h, d = q.shape
    if (k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape or g.shape != q.shape
            or beta.shape != (t, h)):
        raise ValueError("q, k, v, g, dout must be [T, H, D] and beta [T, H]")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv, dg, dbeta = _grad_buffers(grads, q, k, v, g, beta)
    if workspace is None:
        n = kda_bwd_workspace_size(t, nseq, h, d)
        if n == 0:
            raise AttnError(-1, "attn_kda_bwd_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if reuse and check_reuse:
        _check_reuse(workspace, ("kda", t, nseq, h), "attn_kda_bwd_ex(ATTN_DELTA_BWD_REUSE)")
    st = load_library().attn_kda_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(dout), _ptr(cu_seqlens), nseq, t, h, d, float(scale),
                                        1 if reuse else 0, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                        _ptr(dbeta), _ptr(workspace), workspace.numel(),
                                        _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kda_bwd_ex")
    if not reuse:   # the recomputing backward saves into its workspace
        _WS_RECORD[_ws_key(workspace)] = ("kda", t, nseq, h)
    return dq, dk, dv, dg, dbeta


def delta_bwd_workspace_size(total_tokens: int, num_seqs: int, num_heads: int,
                             head_dim: int) -> int:
    return int(load_library().attn_delta_bwd_workspace_size(total_tokens, num_seqs, num_heads,
                                                             head_dim))


def delta_bwd(q, k, v, g, beta, dout, cu_seqlens, scale: float | None = None, workspace=None,
              reuse: bool = False, check_reuse: bool = True, grads=None):
    """attn_delta_bwd(_ex): gradients of sum(dout * out) of the gated
    delta-rule forward.  Returns dq, dk, dv (bf16 [T, H, D]) and dg, dbeta
    (fp32 [T, H]), zero-filled first.  reuse=True takes the records and states
    a delta_fwd(..., save=True) with the same inputs left in `workspace`."""
    if reuse and workspace is None:
        raise ValueError("reuse needs the workspace of a saving forward")
    for name, t_ in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_tensor(name, t_, torch.bfloat16, 3)
    _check_tensor("g", g, torch.float32, 2)
    _check_tensor("beta", beta, torch.float32, 2)
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    t, h, d = q.shape
    if (k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape
            or g.shape != (t, h) or beta.shape != (t, h)):
        raise ValueError("q, k, v, dout must be [T, H, D] and g, beta [T, H]")
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv, dg, dbeta = _grad_buffers(grads, q, k, v, g, beta)
    if workspace is None:
        n = delta_bwd_workspace_size(t, nseq, h, d)
        if n == 0:
            raise AttnError(-1, "attn_delta_bwd_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if reuse and check_reuse:
        _check_reuse(workspace, ("delta", t, nseq, h), "attn_delta_bwd_ex(ATTN_DELTA_BWD_REUSE)")
    st = load_library().attn_delta_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(dout), _ptr(cu_seqlens), nseq, t, h, d,
                                          float(scale), 1 if reuse else 0, _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(workspace),
                                          workspace.numel(), _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_delta_bwd_ex")
    if not reuse:   # the recomputing backward saves into its workspace
        _WS_RECORD[_ws_key(workspace)] = ("delta", t, nseq, h)
    return dq, dk, dv, dg, dbeta


def profile_start() -> None:
    """Bracket every following kernel launch with HIP events on its stream."""
    st = load_library().attn_varlen_profile_start()
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_profile_start")


def profile_stop() -> dict:
    """Stop recording; {kernel: {launches, total_ms, avg_ms, min_ms, max_ms}}."""
    buf = (KernelStats * 16)()
    n = load_library().attn_varlen_profile_stop(buf, 16)
    if n < 0:
        raise AttnError(n, "attn_varlen_profile_stop")
    res = {}
    for s_ in buf[:min(n, 16)]:
        res[s_.name.decode()] = {"launches": s_.launches, "total_ms": s_.total_ms,
                                 "avg_ms": s_.total_ms / max(s_.launches, 1),
                                 "min_ms": s_.min_ms, "max_ms": s_.max_ms}
    return res
