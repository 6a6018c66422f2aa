"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an oracle module (``oracle.attention`` or a
deliberately broken copy of it) and raises AssertionError when the module
disagrees with a closed form, an identity of the mathematics, a textbook
library routine, or a hand-derived worked example.  ``test_oracle_pins``
runs them on the real oracle; ``test_oracle_mutations`` runs them on copies
with a plausible mistake planted and requires that one of them fails.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_3tok.json")


def rand_inputs(seed, cu, hq, hkv, d, scale_q=1.0):
    rng = np.random.default_rng(seed)
    t = int(cu[-1])
    q = rng.standard_normal((t, hq, d)) * scale_q
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    do = rng.standard_normal((t, hq, d))
    return q, k, v, do


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


# --------------------------------------------------------------------------
# Hand-derived worked example (tests/golden/closed_form_3tok.json)
# --------------------------------------------------------------------------
def pin_golden(o):
    g = json.load(open(GOLDEN))
    inp = g["inputs"]
    q = np.array(inp["q"], dtype=np.float64)
    k = np.array(inp["k"], dtype=np.float64)
    v = np.array(inp["v"], dtype=np.float64)
    do = np.array(inp["dout"], dtype=np.float64)
    scale = math.log(3.0)
    frac = np.vectorize(lambda s: float(Fraction(s)))
    logs = np.vectorize(lambda s: math.log(int(s[2:])))
    for name, c in g["cases"].items():
        out, lse = o.attention_forward(q, k, v, inp["cu_seqlens"], c["window"], scale)
        dq, dk, dv, out2, lse2, _ = o.attention_backward(q, k, v, do, inp["cu_seqlens"],
                                                         c["window"], scale)
        _close(out, frac(np.array(c["out"])), 1e-12, f"golden {name} out")
        _close(out2, out, 0, f"golden {name} out (bwd)")
        _close(lse, logs(np.array(c["lse"])), 1e-12, f"golden {name} lse")
        _close(dq / scale, frac(np.array(c["dq_over_ln3"])), 1e-12, f"golden {name} dq")
        _close(dk / scale, frac(np.array(c["dk_over_ln3"])), 1e-12, f"golden {name} dk")
        _close(dv, frac(np.array(c["dv"])), 1e-12, f"golden {name} dv")


# --------------------------------------------------------------------------
# Invariants and closed forms
# --------------------------------------------------------------------------
CU_MIXED = [0, 1, 6, 6, 13, 14, 29, 37]      # 1-token docs, an empty doc, odd lengths


def pin_rows_sum_to_one(o):
    """With v = 1 every output is 1 (softmax rows sum to 1) for every window."""
    q, k, v, _ = rand_inputs(1, CU_MIXED, 4, 2, 8, 2.0)
    v = np.ones_like(v)
    for w in (0, 1, 3, 8):
        out, lse = o.attention_forward(q, k, v, CU_MIXED, w, 0.7)
        _close(out, np.ones_like(out), 1e-12, f"rows sum to 1 (W={w})")
        assert np.all(np.isfinite(lse))


def pin_one_token_document(o):
    """A 1-token document: O = v, LSE = S_ii, dq = dk = 0, dv = sum of group dO."""
    cu = [0, 4, 5, 9]                           # token 4 is a document alone
    q, k, v, do = rand_inputs(2, cu, 4, 2, 8)
    scale = 0.5
    for w in (0, 2):
        dq, dk, dv, out, lse, _ = o.attention_backward(q, k, v, do, cu, w, scale)
        for h in range(4):
            g = h // 2
            _close(out[4, h], v[4, g], 1e-12, "1-token O = v")
            _close(lse[h, 4], scale * q[4, h] @ k[4, g], 1e-12, "1-token LSE = S_ii")
            _close(dq[4, h], np.zeros(8), 1e-12, "1-token dq = 0")
        for g in range(2):
            _close(dk[4, g], np.zeros(8), 1e-12, "1-token dk = 0")
            _close(dv[4, g], do[4, 2 * g] + do[4, 2 * g + 1], 1e-12, "1-token dv")


def pin_q_zero_uniform(o):
    """q = 0: P is uniform over the visible keys, so O is their mean and
    LSE = log(number of visible keys) = log(min(i - a + 1, W))."""
    cu = [0, 5, 17, 18, 30]
    _, k, v, _ = rand_inputs(3, cu, 2, 1, 4)
    q = np.zeros((30, 2, 4))
    for w in (0, 1, 3, 7):
        out, lse = o.attention_forward(q, k, v, cu, w, 1.3)
        for a, b in zip(cu[:-1], cu[1:]):
            for i in range(a, b):
                lo = a if w <= 0 else max(a, i - w + 1)
                n = i - lo + 1
                for h in range(2):
                    _close(lse[h, i], math.log(n), 1e-12, f"q=0 LSE (W={w}, i={i})")
                    _close(out[i, h], v[lo:i + 1, 0].mean(axis=0), 1e-12, f"q=0 O (W={w})")


def pin_window_ge_length_is_global(o):
    """Window >= longest segment equals full causal context, bitwise."""
    q, k, v, do = rand_inputs(4, CU_MIXED, 4, 2, 8)
    ref = o.attention_backward(q, k, v, do, CU_MIXED, 0, 0.3)
    for w in (15, 16, 100):
        got = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.3)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"window {w} differs from global"


def pin_split_document(o):
    """[0, a, a+b] equals the two documents run on their own."""
    a, b = 7, 11
    q, k, v, do = rand_inputs(5, [0, a + b], 4, 2, 8)
    for w in (0, 4):
        whole = o.attention_backward(q, k, v, do, [0, a, a + b], w, 0.4)
        left = o.attention_backward(q[:a], k[:a], v[:a], do[:a], [0, a], w, 0.4)
        right = o.attention_backward(q[a:], k[a:], v[a:], do[a:], [0, b], w, 0.4)
        for x, l, r, name in zip(whole, left, right, ("dq", "dk", "dv", "out", "lse", "D")):
            axis = 1 if name in ("lse", "D") else 0
            _close(x, np.concatenate([l, r], axis=axis), 1e-12, f"split doc {name} (W={w})")


def pin_gqa_is_repeated_mha(o):
    """GQA equals MHA with each kv head repeated G times; dk, dv are group sums."""
    cu = [0, 9, 20]
    q, k, v, do = rand_inputs(6, cu, 6, 2, 8)
    for w in (0, 3):
        dq, dk, dv, out, lse, _ = o.attention_backward(q, k, v, do, cu, w, 0.35)
        kr = np.repeat(k, 3, axis=1)
        vr = np.repeat(v, 3, axis=1)
        dq2, dk2, dv2, out2, lse2, _ = o.attention_backward(q, kr, vr, do, cu, w, 0.35)
        _close(out, out2, 1e-12, "gqa out")
        _close(lse, lse2, 1e-12, "gqa lse")
        _close(dq, dq2, 1e-12, "gqa dq")
        _close(dk, dk2.reshape(20, 2, 3, 8).sum(axis=2), 1e-12, "gqa dk group sum")
        _close(dv, dv2.reshape(20, 2, 3, 8).sum(axis=2), 1e-12, "gqa dv group sum")


def pin_empty_segments(o):
    """Empty documents anywhere change nothing, bitwise."""
    cu = [0, 5, 12, 20]
    padded = [0, 0, 5, 5, 5, 12, 20, 20, 20]
    q, k, v, do = rand_inputs(7, cu, 4, 2, 8)
    for w in (0, 3):
        a = o.attention_backward(q, k, v, do, cu, w, 0.3)
        b = o.attention_backward(q, k, v, do, padded, w, 0.3)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), "empty segments changed the result"


def pin_permutation(o):
    """Reordering whole documents reorders the outputs the same way."""
    lens = [4, 9, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = rand_inputs(8, cu, 4, 2, 8)
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    cu_p = np.concatenate([[0], np.cumsum([lens[s] for s in order])])
    for w in (0, 2):
        a = o.attention_backward(q, k, v, do, cu, w, 0.3)
        b = o.attention_backward(q[idx], k[idx], v[idx], do[idx], cu_p, w, 0.3)
        for x, y, name in zip(a, b, ("dq", "dk", "dv", "out", "lse", "D")):
            xp = x[:, idx] if name in ("lse", "D") else x[idx]
            _close(xp, y, 1e-12, f"permutation {name}")


def pin_key_shift(o):
    """k_j -> k_j + c on one document shifts each of its rows' scores by a
    constant: out, dq, dk, dv do not change (sum_j dS_ij = 0)."""
    cu = [0, 6, 15]
    q, k, v, do = rand_inputs(9, cu, 4, 2, 8)
    c = np.random.default_rng(99).standard_normal((2, 8))
    k2 = k.copy()
    k2[6:15] += c[None]
    for w in (0, 4):
        a = o.attention_backward(q, k, v, do, cu, w, 0.3)
        b = o.attention_backward(q, k2, v, do, cu, w, 0.3)
        for x, y, name in zip(a[:4], b[:4], ("dq", "dk", "dv", "out")):
            _close(x, y, 1e-10, f"key shift {name}")


def pin_d_identity(o):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i."""
    q, k, v, do = rand_inputs(10, CU_MIXED, 4, 2, 8)
    for w in (0, 3):
        _, _, _, out, _, dd = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.3)
        _close(dd, np.einsum("thd,thd->ht", do, out), 1e-12, "D = dO.O")


def pin_torch_sdpa(o):
    """One document, no window: torch's own scaled_dot_product_attention
    (fp64, CPU, causal) and its autograd, with kv heads repeated."""
    import torch
    t, hq, hkv, d = 19, 4, 2, 8
    q, k, v, do = rand_inputs(11, [0, t], hq, hkv, d)
    scale = 0.45
    dq, dk, dv, out, lse, _ = o.attention_backward(q, k, v, do, [0, t], 0, scale)
    tq = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
    kr = tk.repeat_interleave(hq // hkv, dim=0)
    vr = tv.repeat_interleave(hq // hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq[None], kr[None], vr[None], is_causal=True, scale=scale)[0]
    ref.backward(torch.tensor(do.transpose(1, 0, 2)))
    _close(out, ref.detach().numpy().transpose(1, 0, 2), 1e-10, "sdpa out")
    _close(dq, tq.grad.numpy().transpose(1, 0, 2), 1e-10, "sdpa dq")
    _close(dk, tk.grad.numpy().transpose(1, 0, 2), 1e-10, "sdpa dk")
    _close(dv, tv.grad.numpy().transpose(1, 0, 2), 1e-10, "sdpa dv")
    # LSE through torch's logsumexp over the causal scores
    s = scale * torch.einsum("htd,hsd->hts", tq.detach(), kr.detach())
    s = s.masked_fill(~torch.ones(t, t, dtype=torch.bool).tril(), float("-inf"))
    _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-10, "sdpa lse")


def pin_finite_differences(o):
    """Central differences of loss = sum(dO * O) in fp64 match dq, dk, dv."""
    cu = [0, 1, 9, 9, 20]
    q, k, v, do = rand_inputs(12, cu, 4, 2, 8)
    h = 1e-6
    for w in (0, 3):
        dq, dk, dv, *_ = o.attention_backward(q, k, v, do, cu, w, 0.6)

        def loss(qq, kk, vv):
            out, _ = o.attention_forward(qq, kk, vv, cu, w, 0.6)
            return float((out * do).sum())

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name] = xp
                args_m[name] = xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            r = _rel(grad, num)
            assert r <= 1e-6, f"finite differences d{name} (W={w}): rel err {r:.2e}"


def pin_row_function(o):
    """The single-row function equals the full oracle's row."""
    q, k, v, do = rand_inputs(13, CU_MIXED, 4, 2, 8)
    for w in (0, 3):
        dq, _, _, out, lse, _ = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.3)
        for h, i in ((0, 0), (3, 5), (1, 13), (2, 28), (3, 36)):
            ro, rl, rdq = o.attention_row(q, k, v, do, CU_MIXED, w, 0.3, h, i)
            _close(ro, out[i, h], 1e-12, "row out")
            _close(rl, lse[h, i], 1e-12, "row lse")
            _close(rdq, dq[i, h], 1e-12, "row dq")


# --------------------------------------------------------------------------
# Logit soft-cap: S' = c tanh(S / c) before the softmax
# --------------------------------------------------------------------------
def pin_softcap_two_keys(o):
    """Hand-derived two-key case.  One document [t0, t1], d = 2, scale 1,
    q1 = (2, 0), k0 = (1, 0), k1 = (-1, 0): S_1 = (2, -2) and, with cap
    c = 2, S'_1 = (2 tanh 1, -2 tanh 1).  Row 1 is a two-way softmax:
    p0 = 1 / (1 + exp(-4 tanh 1)), p1 = 1 - p0, LSE = log(2 cosh(2 tanh 1)),
    and dS_10 = -dS_11 = sech^2(1) p0 p1 (dP_10 - dP_11).  Row 0 sees only
    key 0: O_0 = v0, LSE_0 = c tanh(S_00 / c), dS_00 = 0."""
    c = 2.0
    q = np.array([[[0.5, 1.0]], [[2.0, 0.0]]])
    k = np.array([[[1.0, 0.0]], [[-1.0, 0.0]]])
    v = np.array([[[3.0, -1.0]], [[0.5, 2.0]]])
    do = np.array([[[1.0, 2.0]], [[-1.5, 0.25]]])
    dq, dk, dv, out, lse, _ = o.attention_backward(q, k, v, do, [0, 2], 0, 1.0, c)
    th = math.tanh(1.0)
    p0 = 1.0 / (1.0 + math.exp(-4.0 * th))
    p1 = 1.0 - p0
    sech2 = 1.0 - th * th
    dp0 = do[1, 0] @ v[0, 0]
    dp1 = do[1, 0] @ v[1, 0]
    ds10 = sech2 * p0 * p1 * (dp0 - dp1)
    _close(out[0, 0], v[0, 0], 1e-14, "cap 2-key O_0")
    _close(lse[0, 0], c * math.tanh(0.5 / c), 1e-14, "cap 2-key LSE_0")
    _close(out[1, 0], p0 * v[0, 0] + p1 * v[1, 0], 1e-14, "cap 2-key O_1")
    _close(lse[0, 1], math.log(2.0 * math.cosh(2.0 * th)), 1e-14, "cap 2-key LSE_1")
    _close(dq[0, 0], np.zeros(2), 1e-14, "cap 2-key dq_0")
    _close(dq[1, 0], ds10 * (k[0, 0] - k[1, 0]), 1e-14, "cap 2-key dq_1")
    _close(dk[0, 0], ds10 * q[1, 0], 1e-14, "cap 2-key dk_0")
    _close(dk[1, 0], -ds10 * q[1, 0], 1e-14, "cap 2-key dk_1")
    _close(dv[0, 0], do[0, 0] + p0 * do[1, 0], 1e-14, "cap 2-key dv_0")
    _close(dv[1, 0], p1 * do[1, 0], 1e-14, "cap 2-key dv_1")


def pin_softcap_large_is_uncapped(o):
    """c tanh(S / c) = S - S^3 / (3 c^2) + ...: a cap of 1e6 on logits of
    size ~10 changes nothing beyond ~1e-10 relative."""
    q, k, v, do = rand_inputs(14, CU_MIXED, 4, 2, 8, 2.0)
    for w in (0, 3):
        ref = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.6)
        got = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.6, 1e6)
        for x, y, name in zip(got, ref, ("dq", "dk", "dv", "out", "lse", "D")):
            assert _rel(x, y) <= 1e-9, f"cap 1e6 vs none: {name} differs"


def pin_softcap_bounds(o):
    """Every capped logit lies in [-c, c] (tanh reaches +-1 in fp64 once
    saturated), so each row's LSE lies within [log n - c, log n + c] for its
    n visible keys, and rows still sum to one."""
    q, k, v, _ = rand_inputs(15, CU_MIXED, 4, 2, 8, 10.0)
    c = 0.75
    v1 = np.ones_like(v)
    for w in (0, 4):
        out, lse = o.attention_forward(q, k, v1, CU_MIXED, w, 1.0, c)
        _close(out, np.ones_like(out), 1e-12, f"cap rows sum to 1 (W={w})")
        for a, b in zip(CU_MIXED[:-1], CU_MIXED[1:]):
            for i in range(a, b):
                lo = a if w <= 0 else max(a, i - w + 1)
                n = i - lo + 1
                assert np.all(np.abs(lse[:, i] - math.log(n)) <= c + 1e-12), "cap LSE bound"


def pin_softcap_torch_autograd(o):
    """torch (fp64, CPU): scores, tanh cap, masked softmax over a block-
    diagonal causal/window mask, and autograd for the gradients."""
    import torch
    cu = [0, 7, 7, 19, 20, 33]
    hq, hkv, d = 4, 2, 8
    q, k, v, do = rand_inputs(16, cu, hq, hkv, d, 3.0)
    t = cu[-1]
    scale, c = 0.5, 2.5
    for w in (0, 5):
        dq, dk, dv, out, lse, _ = o.attention_backward(q, k, v, do, cu, w, scale, c)
        tq = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
        tk = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)
        tv = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
        kr = tk.repeat_interleave(hq // hkv, dim=0)
        vr = tv.repeat_interleave(hq // hkv, dim=0)
        seg = torch.zeros(t, dtype=torch.long)
        for sidx, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
            seg[a:b] = sidx
        i = torch.arange(t)[:, None]
        j = torch.arange(t)[None, :]
        allowed = (seg[:, None] == seg[None, :]) & (j <= i)
        if w > 0:
            allowed &= j > i - w
        sc = scale * torch.matmul(tq, kr.transpose(1, 2))
        sc = c * torch.tanh(sc / c)
        sc = sc.masked_fill(~allowed, float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=-1)
        ref = torch.matmul(torch.softmax(sc, dim=-1), vr)
        ref.backward(torch.tensor(do.transpose(1, 0, 2)))
        _close(out, ref.detach().numpy().transpose(1, 0, 2), 1e-10, f"cap torch out (W={w})")
        _close(lse, ref_lse.detach().numpy(), 1e-10, f"cap torch lse (W={w})")
        _close(dq, tq.grad.numpy().transpose(1, 0, 2), 1e-10, f"cap torch dq (W={w})")
        _close(dk, tk.grad.numpy().transpose(1, 0, 2), 1e-10, f"cap torch dk (W={w})")
        _close(dv, tv.grad.numpy().transpose(1, 0, 2), 1e-10, f"cap torch dv (W={w})")


def pin_softcap_finite_differences(o):
    """Central differences of sum(dO * O) through the cap (c = 1.5, logits
    of size ~5, so tanh is far from linear)."""
    cu = [0, 1, 6, 13]
    q, k, v, do = rand_inputs(17, cu, 2, 1, 4, 2.0)
    h = 1e-6
    c, scale = 1.5, 0.8
    for w in (0, 3):
        dq, dk, dv, *_ = o.attention_backward(q, k, v, do, cu, w, scale, c)

        def loss(qq, kk, vv):
            out, _ = o.attention_forward(qq, kk, vv, cu, w, scale, c)
            return float((out * do).sum())

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name] = x.copy()
                args_m[name] = x.copy()
                args_p[name][idx] += h
                args_m[name][idx] -= h
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            r = _rel(grad, num)
            assert r <= 1e-6, f"cap finite differences d{name} (W={w}): rel err {r:.2e}"


def pin_softcap_row_function(o):
    """The single-row function equals the full oracle's row, with a cap."""
    q, k, v, do = rand_inputs(18, CU_MIXED, 4, 2, 8, 2.0)
    for w in (0, 3):
        dq, _, _, out, lse, _ = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.3, 1.25)
        for h, i in ((0, 0), (3, 5), (1, 13), (2, 28), (3, 36)):
            ro, rl, rdq = o.attention_row(q, k, v, do, CU_MIXED, w, 0.3, h, i, 1.25)
            _close(ro, out[i, h], 1e-12, "cap row out")
            _close(rl, lse[h, i], 1e-12, "cap row lse")
            _close(rdq, dq[i, h], 1e-12, "cap row dq")


def pin_key_function(o):
    """The single-key function equals the full oracle's dk, dv rows (with and
    without a window and a cap), for keys at segment starts, ends and inside."""
    q, k, v, do = rand_inputs(19, CU_MIXED, 4, 2, 8, 1.5)
    for w, cap in ((0, 0.0), (3, 0.0), (4, 1.25)):
        _, dk, dv, *_ = o.attention_backward(q, k, v, do, CU_MIXED, w, 0.3, cap)
        for g, j in ((0, 0), (1, 5), (0, 6), (1, 12), (0, 13), (1, 14), (0, 28), (1, 36)):
            rk, rv = o.attention_key(q, k, v, do, CU_MIXED, w, 0.3, g, j, cap)
            _close(rk, dk[j, g], 1e-12, f"key dk (W={w}, cap={cap}, j={j})")
            _close(rv, dv[j, g], 1e-12, f"key dv (W={w}, cap={cap}, j={j})")


ALL_PINS = [
    pin_golden,
    pin_rows_sum_to_one,
    pin_one_token_document,
    pin_q_zero_uniform,
    pin_window_ge_length_is_global,
    pin_split_document,
    pin_gqa_is_repeated_mha,
    pin_empty_segments,
    pin_permutation,
    pin_key_shift,
    pin_d_identity,
    pin_row_function,
    pin_key_function,
    pin_torch_sdpa,
    pin_finite_differences,
    pin_softcap_two_keys,
    pin_softcap_large_is_uncapped,
    pin_softcap_bounds,
    pin_softcap_row_function,
    pin_softcap_torch_autograd,
    pin_softcap_finite_differences,
]


# --------------------------------------------------------------------------
# Band-block formulation (oracle/band.py): pinned against the dense oracle
# (itself pinned above) and against closed forms of its own.
# --------------------------------------------------------------------------
BAND_CASES = [(CU_MIXED, 1), (CU_MIXED, 3), (CU_MIXED, 8), ([0, 40, 70], 7),
              ([0, 5, 64], 16), ([0, 3, 3, 19, 52], 5), (CU_MIXED, 40)]


def pin_band_equals_dense(ob):
    """Band-block results equal the dense definition (windows of 1 key up to
    longer than the microbatch, blocks crossing document boundaries)."""
    from oracle import attention as dense
    for n, (cu, w) in enumerate(BAND_CASES):
        q, k, v, do = rand_inputs(40 + n, cu, 4, 2, 8, 1.2)
        out, lse, dq, dk, dv = ob.band_attention(q, k, v, do, cu, w, 0.35)
        rdq, rdk, rdv, rout, rlse, _ = dense.attention_backward(q, k, v, do, cu, w, 0.35)
        for name, x, y in (("out", out, rout), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            _close(x, y, 1e-11, f"band {name} (W={w}, cu={cu})")
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(lse), fin), f"band lse support (W={w})"
        _close(lse[fin], rlse[fin], 1e-11, f"band lse (W={w})")


def pin_band_bias_counts(ob):
    """Row i of a band sees exactly min(i - a + 1, W) keys (a its segment
    start), all inside the band's [(b - 1) W, (b + 1) W) columns."""
    cu = [0, 3, 3, 19, 52]
    for w in (1, 4, 7, 20, 60):
        t = cu[-1]
        for b in range((t + w - 1) // w):
            q0, q1, lo, hi, bias = ob.band_bias(cu, t, w, b)
            assert (q0, q1, lo, hi) == (b * w, min(t, (b + 1) * w), max(0, (b - 1) * w), min(t, (b + 1) * w))
            assert bias.shape == (q1 - q0, hi - lo)
            for r, i in enumerate(range(q0, q1)):
                a = cu[int(np.searchsorted(cu, i, side="right")) - 1]   # start of i's segment
                want = min(i - a + 1, w)
                got = int(np.isfinite(bias[r]).sum())
                assert got == want, f"band row {i} (W={w}): {got} visible keys, want {want}"


def pin_band_q_zero(ob):
    """q = 0 makes every visible key equally likely: lse = log(min(i - a + 1, W))
    and out = the mean of the visible values (closed form)."""
    cu = [0, 9, 30]
    w = 6
    _, k, v, do = rand_inputs(47, cu, 4, 2, 8)
    q = np.zeros((cu[-1], 4, 8))
    out, lse, *_ = ob.band_attention(q, k, v, do, cu, w, 0.5)
    for a, b in ((0, 9), (9, 30)):
        for i in range(a, b):
            lo = max(a, i - w + 1)
            for h in range(4):
                assert abs(lse[h, i] - math.log(i - lo + 1)) <= 1e-12, f"band lse row {i}"
                _close(out[i, h], v[lo:i + 1, h // 2].mean(axis=0), 1e-12, f"band out row {i}")


BAND_PINS = [pin_band_equals_dense, pin_band_bias_counts, pin_band_q_zero]
