"""Checks that pin the gated delta-rule oracle (oracle/delta.py) to closed
forms and to finite differences.  Each ``pin_*`` takes an oracle module (the
real one or a copy with a planted mistake) and raises AssertionError on a
disagreement; tests/test_oracle_delta.py runs them."""
from __future__ import annotations

import numpy as np


def _inputs(seed, cu, h, dk, dv, beta_range=(0.1, 0.9), g_range=(-0.7, 0.0)):
    rng = np.random.default_rng(seed)
    t = int(cu[-1])
    q = rng.standard_normal((t, h, dk))
    k = rng.standard_normal((t, h, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)          # unit keys, as the model feeds them
    v = rng.standard_normal((t, h, dv))
    g = rng.uniform(*g_range, size=(t, h))
    beta = rng.uniform(*beta_range, size=(t, h))
    return q, k, v, g, beta


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def pin_delta_no_write(od):
    """beta = 0: nothing is ever written, every output is exactly zero."""
    cu = [0, 5, 12]
    q, k, v, g, _ = _inputs(1, cu, 2, 4, 3)
    o = od.gated_delta_forward(q, k, v, g, np.zeros_like(g), cu, 0.7)
    assert np.all(o == 0.0), "beta = 0 wrote into the state"


def pin_delta_single_token_documents(od):
    """One-token documents: S_1 = beta v k^T, so o = scale beta (k . q) v."""
    cu = np.arange(0, 7)
    q, k, v, g, beta = _inputs(2, cu, 2, 4, 3)
    o = od.gated_delta_forward(q, k, v, g, beta, cu, 0.6)
    want = 0.6 * beta[..., None] * np.einsum("thd,thd->th", k, q)[..., None] * v
    _close(o, want, 1e-12, "one-token documents")


def pin_delta_overwrite(od):
    """alpha = 1, beta = 1 and keys cycling through the unit vectors: each
    write replaces one column of S, so o_t = scale sum_j q_t[j] v_last(j)."""
    dk, dv = 4, 3
    cu = [0, 9, 15]
    rng = np.random.default_rng(3)
    t = cu[-1]
    q = rng.standard_normal((t, 1, dk))
    v = rng.standard_normal((t, 1, dv))
    k = np.zeros((t, 1, dk))
    for a, b in zip(cu[:-1], cu[1:]):
        for i in range(a, b):
            k[i, 0, (i - a) % dk] = 1.0
    o = od.gated_delta_forward(q, k, v, np.zeros((t, 1)), np.ones((t, 1)), cu, 0.5)
    for a, b in zip(cu[:-1], cu[1:]):
        last = {}
        for i in range(a, b):
            last[(i - a) % dk] = v[i, 0]
            want = 0.5 * sum(q[i, 0, j] * vec for j, vec in last.items())
            _close(o[i, 0], want, 1e-12, f"overwrite row {i}")


def pin_delta_decay(od):
    """Orthonormal keys within a document (no interference) with constant
    decay alpha and strength beta: S_t = sum_i alpha^(t-i) beta v_i k_i^T."""
    dk, dv = 6, 2
    cu = [0, 6, 10]
    rng = np.random.default_rng(4)
    t = cu[-1]
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    q = rng.standard_normal((t, 1, dk))
    v = rng.standard_normal((t, 1, dv))
    k = np.zeros((t, 1, dk))
    for a, b in zip(cu[:-1], cu[1:]):
        for i in range(a, b):
            k[i, 0] = basis[i - a]
    alpha, beta = 0.8, 0.35
    o = od.gated_delta_forward(q, k, v, np.full((t, 1), np.log(alpha)), np.full((t, 1), beta), cu, 1.0)
    for a, b in zip(cu[:-1], cu[1:]):
        for i in range(a, b):
            want = sum(alpha ** (i - j) * beta * (k[j, 0] @ q[i, 0]) * v[j, 0] for j in range(a, i + 1))
            _close(o[i, 0], want, 1e-12, f"decay row {i}")


def pin_delta_documents_independent(od):
    """Two documents in one microbatch give the two separate results."""
    cu = [0, 7, 16]
    q, k, v, g, beta = _inputs(5, cu, 2, 5, 4)
    o = od.gated_delta_forward(q, k, v, g, beta, cu, 0.4)
    o1 = od.gated_delta_forward(q[:7], k[:7], v[:7], g[:7], beta[:7], [0, 7], 0.4)
    o2 = od.gated_delta_forward(q[7:], k[7:], v[7:], g[7:], beta[7:], [0, 9], 0.4)
    _close(o, np.concatenate([o1, o2]), 1e-13, "document split")


def pin_delta_backward_matches_forward(od):
    """The backward's recomputed output equals the forward's."""
    cu = [0, 4, 11]
    q, k, v, g, beta = _inputs(6, cu, 2, 5, 3)
    do = np.random.default_rng(7).standard_normal((11, 2, 3))
    *_, o = od.gated_delta_backward(q, k, v, g, beta, do, cu, 0.3)
    _close(o, od.gated_delta_forward(q, k, v, g, beta, cu, 0.3), 1e-13, "backward's output")


def pin_delta_finite_differences(od):
    """Central differences of sum(dout * o) for every input (float64)."""
    cu = [0, 3, 7]
    q, k, v, g, beta = _inputs(8, cu, 2, 3, 2)
    do = np.random.default_rng(9).standard_normal((7, 2, 2))
    grads = od.gated_delta_backward(q, k, v, g, beta, do, cu, 0.8)[:5]
    args = [q, k, v, g, beta]
    eps = 1e-6
    for idx, name in enumerate(("q", "k", "v", "g", "beta")):
        x = args[idx]
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            for sgn in (1, -1):
                xs = [a.copy() for a in args]
                xs[idx][pos] += sgn * eps
                f = float(np.sum(do * od.gated_delta_forward(*xs, cu, 0.8)))
                num[pos] += sgn * f / (2 * eps)
        err = np.max(np.abs(num - grads[idx])) / max(1.0, np.max(np.abs(num)))
        assert err <= 1e-6, f"d{name}: finite-difference mismatch {err:.2e}"


DELTA_PINS = [pin_delta_no_write, pin_delta_single_token_documents, pin_delta_overwrite,
              pin_delta_decay, pin_delta_documents_independent,
              pin_delta_backward_matches_forward, pin_delta_finite_differences]
