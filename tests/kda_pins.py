"""Checks that pin the Kimi Delta Attention oracle (oracle/kimi_delta.py):
the Gated DeltaNet oracle when every channel has the same gate, independent
per-column recurrences when the keys are coordinate axes, closed forms and
finite differences.  Each ``pin_*`` takes an oracle module (the real one or
a copy with a planted mistake) and raises AssertionError on a disagreement;
tests/test_oracle_kimi_delta.py runs them."""
from __future__ import annotations

import numpy as np

from oracle import delta as gdn


def _inputs(seed, cu, h, dk, dv, beta_range=(0.1, 0.9), g_range=(-0.7, 0.0)):
    rng = np.random.default_rng(seed)
    t = int(cu[-1])
    q = rng.standard_normal((t, h, dk))
    k = rng.standard_normal((t, h, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((t, h, dv))
    g = rng.uniform(*g_range, size=(t, h, dk))
    beta = rng.uniform(*beta_range, size=(t, h))
    return q, k, v, g, beta


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def pin_kda_no_write(ok):
    """beta = 0: nothing is written, every output is exactly zero."""
    cu = [0, 5, 12]
    q, k, v, g, _ = _inputs(1, cu, 2, 4, 3)
    o = ok.kimi_delta_forward(q, k, v, g, np.zeros((12, 2)), cu, 0.7)
    assert np.all(o == 0.0), "beta = 0 wrote into the state"


def pin_kda_single_token_documents(ok):
    """One-token documents: S_1 = beta v k^T, so o = scale beta (k . q) v."""
    cu = np.arange(0, 7)
    q, k, v, g, beta = _inputs(2, cu, 2, 4, 3)
    o = ok.kimi_delta_forward(q, k, v, g, beta, cu, 0.6)
    want = 0.6 * beta[..., None] * np.einsum("thd,thd->th", k, q)[..., None] * v
    _close(o, want, 1e-12, "one-token documents")


def pin_kda_equal_channels_is_gdn(ok):
    """A gate equal on every key channel is Gated DeltaNet's scalar gate."""
    cu = [0, 9, 9, 20]
    q, k, v, g, beta = _inputs(3, cu, 2, 5, 4)
    gs = g[..., 0]
    o = ok.kimi_delta_forward(q, k, v, np.repeat(gs[..., None], 5, axis=-1), beta, cu, 0.45)
    _close(o, gdn.gated_delta_forward(q, k, v, gs, beta, cu, 0.45), 1e-12, "equal channels")


def pin_kda_axis_keys(ok):
    """Keys on coordinate axes (k_t = e_c): column c of S follows
    col <- (1 - beta) alpha_c col + beta v, every other column d just decays
    by alpha_d, and o = scale sum_c q_c col_c.  Here d_v = d_k, so a gate on
    the wrong axis fails numerically rather than by shape."""
    dk = dv = 4
    cu = [0, 11, 18]
    rng = np.random.default_rng(4)
    t = cu[-1]
    q = rng.standard_normal((t, 1, dk))
    v = rng.standard_normal((t, 1, dv))
    g = rng.uniform(-0.9, -0.05, size=(t, 1, dk))
    beta = rng.uniform(0.2, 0.9, size=(t, 1))
    axis = rng.integers(0, dk, size=t)
    k = np.zeros((t, 1, dk))
    k[np.arange(t), 0, axis] = 1.0
    o = ok.kimi_delta_forward(q, k, v, g, beta, cu, 0.9)
    for a, b in zip(cu[:-1], cu[1:]):
        cols = [np.zeros(dv) for _ in range(dk)]
        for i in range(a, b):
            alpha = np.exp(g[i, 0])
            for c in range(dk):
                if c == axis[i]:
                    cols[c] = (1 - beta[i, 0]) * alpha[c] * cols[c] + beta[i, 0] * v[i, 0]
                else:
                    cols[c] = alpha[c] * cols[c]
            want = 0.9 * sum(q[i, 0, c] * cols[c] for c in range(dk))
            _close(o[i, 0], want, 1e-12, f"axis keys row {i}")


def pin_kda_documents_independent(ok):
    """Two documents in one microbatch give the two separate results."""
    cu = [0, 7, 16]
    q, k, v, g, beta = _inputs(5, cu, 2, 5, 4)
    o = ok.kimi_delta_forward(q, k, v, g, beta, cu, 0.4)
    o1 = ok.kimi_delta_forward(q[:7], k[:7], v[:7], g[:7], beta[:7], [0, 7], 0.4)
    o2 = ok.kimi_delta_forward(q[7:], k[7:], v[7:], g[7:], beta[7:], [0, 9], 0.4)
    _close(o, np.concatenate([o1, o2]), 1e-13, "document split")


def pin_kda_backward_matches_forward(ok):
    """The backward's recomputed output equals the forward's."""
    cu = [0, 4, 11]
    q, k, v, g, beta = _inputs(6, cu, 2, 5, 3)
    do = np.random.default_rng(7).standard_normal((11, 2, 3))
    *_, o = ok.kimi_delta_backward(q, k, v, g, beta, do, cu, 0.3)
    _close(o, ok.kimi_delta_forward(q, k, v, g, beta, cu, 0.3), 1e-13, "backward's output")


def pin_kda_finite_differences(ok):
    """Central differences of sum(dout * o) for every input, the per-channel
    gate included (float64)."""
    cu = [0, 3, 7]
    q, k, v, g, beta = _inputs(8, cu, 2, 3, 2)
    do = np.random.default_rng(9).standard_normal((7, 2, 2))
    grads = ok.kimi_delta_backward(q, k, v, g, beta, do, cu, 0.8)[:5]
    args = [q, k, v, g, beta]
    eps = 1e-6
    for idx, name in enumerate(("q", "k", "v", "g", "beta")):
        x = args[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            for sgn in (1, -1):
                xs = [a.copy() for a in args]
                xs[idx][pos] += sgn * eps
                f = float(np.sum(do * ok.kimi_delta_forward(*xs, cu, 0.8)))
                num[pos] += sgn * f / (2 * eps)
        err = np.max(np.abs(num - grads[idx])) / max(1.0, np.max(np.abs(num)))
        assert err <= 1e-6, f"d{name}: finite-difference mismatch {err:.2e}"


KDA_PINS = [pin_kda_no_write, pin_kda_single_token_documents, pin_kda_equal_channels_is_gdn,
            pin_kda_axis_keys, pin_kda_documents_independent, pin_kda_backward_matches_forward,
            pin_kda_finite_differences]
