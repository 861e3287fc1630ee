"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin compares the oracle with something fixed independently of its code:
hand-derived closed forms (tests/golden/hand_cases.json), brute force on tiny
inputs with scalar loops, closed forms for special inputs (identical keys,
constant values, the first causal row), invariants (rows of P sum to one,
shift invariance, gradient sums), central finite differences of the loss
sum(O * dO), and torch's own CPU attention and autograd in float64.

The last test plants plausible mistakes in copies of the oracle's source and
checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ----------------------------------------------------------------- helpers --

def _expr(s: str) -> float:
    """Evaluate a golden-file expression: a rational, ln(x), or a*ln(x)."""
    s = s.strip()
    if s in ("-inf", "inf"):
        return float(s)
    if "*ln(" in s:
        a, b = s.split("*ln(")
        return float(Fraction(a)) * math.log(float(Fraction(b[:-1])))
    if s.startswith("ln("):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(nested) -> np.ndarray:
    if isinstance(nested, str):
        return np.array(_expr(nested))
    return np.array([_arr(x) for x in nested])


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _brute_fwd(q, k, v, scale, causal, window=(-1, -1)):
    """Scalar-loop attention straight from the definition (tiny sizes only)."""
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    g = hq // hkv
    o = np.zeros((B, nq, hq, d))
    lse = np.zeros((B, hq, nq))
    for b in range(B):
        for h in range(hq):
            kh = h // g
            for i in range(nq):
                scores = []
                for j in range(nk):
                    if causal and j > i + (nk - nq):
                        continue
                    if window[0] >= 0 and j < i + (nk - nq) - window[0]:
                        continue
                    if window[1] >= 0 and j > i + (nk - nq) + window[1]:
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += q[b, i, h, c] * k[b, j, kh, c]
                    scores.append((j, scale * dot))
                if not scores:
                    lse[b, h, i] = -math.inf
                    continue
                total = sum(math.exp(sv) for _, sv in scores)
                lse[b, h, i] = math.log(total)
                for j, sv in scores:
                    w = math.exp(sv) / total
                    for c in range(d):
                        o[b, i, h, c] += w * v[b, j, kh, c]
    return o, lse


# ------------------------------------------------------------- pin checks --
# Each check takes the oracle module (or a mutant of it) and raises
# AssertionError when the pin does not hold.

def pin_golden_fwd(m):
    data = json.load(open(GOLDEN))
    for case in data["fwd"]:
        q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
        scale = _expr(case["scale"])
        for mode, causal in (("causal", True), ("noncausal", False)):
            o, lse = m.attn_fwd(q, k, v, scale, causal)
            np.testing.assert_allclose(o, _arr(case[mode]["o"]), rtol=0, atol=1e-13, err_msg=case["name"] + mode)
            np.testing.assert_allclose(lse, _arr(case[mode]["lse"]), rtol=0, atol=1e-13, err_msg=case["name"] + mode)


def pin_golden_bwd(m):
    data = json.load(open(GOLDEN))
    for case in data["bwd"]:
        args = [_arr(case[n]) for n in ("q", "k", "v", "do")]
        dq, dk, dv, _ = m.attn_bwd(*args, _expr(case["scale"]), case["causal"])
        np.testing.assert_allclose(dq, _arr(case["dq"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, _arr(case["dk"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, _arr(case["dv"]), rtol=0, atol=1e-13)


def pin_golden_decode(m):
    data = json.load(open(GOLDEN))
    for case in data["decode"]:
        o, lse = m.attn_decode(_arr(case["q"]), _arr(case["k_cache"]), _arr(case["v_cache"]),
                               np.array(case["cache_seqlens"]), _expr(case["scale"]))
        np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-13)


BRUTE_SHAPES = [
    # B, Nq, Nk, Hq, Hkv, d
    (1, 1, 1, 1, 1, 1),
    (1, 5, 5, 1, 1, 3),
    (2, 8, 8, 4, 2, 4),
    (1, 3, 7, 2, 1, 5),
    (1, 6, 6, 3, 3, 8),
    (2, 4, 4, 8, 1, 2),
]


def pin_brute_force(m):
    rng = np.random.default_rng(1)
    for (B, nq, nk, hq, hkv, d) in BRUTE_SHAPES:
        q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
        scale = 0.37 + 0.1 * d
        for causal in (False, True):
            o, lse = m.attn_fwd(q, k, v, scale, causal)
            ob, lb = _brute_fwd(q, k, v, scale, causal)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def pin_identical_keys(m):
    """All keys equal: O_i is the mean of the visible V rows, LSE_i = s_i + ln n_i."""
    rng = np.random.default_rng(2)
    B, N, H, d = 2, 9, 2, 4
    q = _rand(rng, B, N, H, d)
    krow = _rand(rng, d)
    k = np.broadcast_to(krow, (B, N, H, d)).copy()
    v = _rand(rng, B, N, H, d)
    scale = 0.5
    for causal in (False, True):
        o, lse = m.attn_fwd(q, k, v, scale, causal)
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(o[:, i], v[:, :n].mean(axis=1), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[:, :, i], scale * q[:, i] @ krow + math.log(n), rtol=0, atol=1e-13)
        # with Q = 0 the logsumexp is exactly ln n
        _, lse0 = m.attn_fwd(np.zeros_like(q), k, v, scale, causal)
        n = np.arange(1, N + 1) if causal else np.full(N, N)
        np.testing.assert_allclose(lse0, np.broadcast_to(np.log(n), lse0.shape), rtol=0, atol=1e-14)


def pin_first_causal_row(m):
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 2, 7, 4, 5), _rand(rng, 2, 7, 2, 5), _rand(rng, 2, 7, 2, 5)
    o, lse = m.attn_fwd(q, k, v, 0.3, True)
    for h in range(4):
        np.testing.assert_array_equal(o[:, 0, h], v[:, 0, h // 2])
        np.testing.assert_allclose(lse[:, h, 0], 0.3 * np.einsum("bc,bc->b", q[:, 0, h], k[:, 0, h // 2]), rtol=0, atol=1e-14)


def pin_rows_sum_to_one(m):
    rng = np.random.default_rng(4)
    q, k = _rand(rng, 6, 5), _rand(rng, 9, 5)
    for causal in (False, True):
        s, p, _ = m.head_probs(q, k, 0.8, causal)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (p >= 0).all()
        if causal:
            masked = np.arange(9)[None, :] > np.arange(6)[:, None] + 3
            assert (p[masked] == 0).all() and np.isneginf(s[masked]).all()
            assert (p[~masked] > 0).all()


def pin_shift_invariance(m):
    """K_j += c for every j leaves O unchanged and shifts LSE_i by scale q_i . c."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 6, 2, 3), _rand(rng, 1, 6, 1, 3), _rand(rng, 1, 6, 1, 3)
    c = np.array([2.0, -1.0, 0.5])
    for causal in (False, True):
        o1, l1 = m.attn_fwd(q, k, v, 0.7, causal)
        o2, l2 = m.attn_fwd(q, k + c, v, 0.7, causal)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, 0.7 * np.einsum("bihc,c->bhi", q, c), rtol=0, atol=1e-12)


def pin_value_tests(m):
    rng = np.random.default_rng(6)
    q, k = _rand(rng, 1, 5, 2, 3), _rand(rng, 1, 5, 2, 3)
    const = np.array([1.5, -2.0, 0.25])
    v = np.broadcast_to(const, (1, 5, 2, 3)).copy()
    for causal in (False, True):
        o, _ = m.attn_fwd(q, k, v, 1.1, causal)
        np.testing.assert_allclose(o, np.broadcast_to(const, o.shape), rtol=0, atol=1e-14)
        v1, v2 = _rand(rng, 1, 5, 2, 3), _rand(rng, 1, 5, 2, 3)
        oa, _ = m.attn_fwd(q, k, 2.0 * v1 - 3.0 * v2, 1.1, causal)
        ob1, _ = m.attn_fwd(q, k, v1, 1.1, causal)
        ob2, _ = m.attn_fwd(q, k, v2, 1.1, causal)
        np.testing.assert_allclose(oa, 2.0 * ob1 - 3.0 * ob2, rtol=0, atol=1e-12)


def pin_finite_differences(m):
    rng = np.random.default_rng(7)
    shapes = [(1, 4, 4, 2, 1, 3), (1, 3, 5, 2, 2, 2)]
    h = 1e-6
    for (B, nq, nk, hq, hkv, d) in shapes:
        q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
        do = _rand(rng, B, nq, hq, d)
        for causal in (False, True):
            dq, dk, dv, _ = m.attn_bwd(q, k, v, do, 0.6, causal)

            def loss(qq, kk, vv):
                return float((m.attn_fwd(qq, kk, vv, 0.6, causal)[0] * do).sum())

            for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
                num = np.zeros_like(x)
                it = np.nditer(x, flags=["multi_index"])
                for _ in it:
                    idx = it.multi_index
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += h
                    xm[idx] -= h
                    args_p = {"q": q, "k": k, "v": v}
                    args_m = dict(args_p)
                    args_p[name], args_m[name] = xp, xm
                    num[idx] = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                                - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * h)
                err = np.abs(num - grad).max() / max(1.0, np.abs(grad).max())
                assert err < 1e-6, (name, causal, err)


def pin_gradient_invariants(m):
    rng = np.random.default_rng(8)
    B, N, hq, hkv, d = 2, 16, 4, 2, 8
    q, k, v, do = _rand(rng, B, N, hq, d), _rand(rng, B, N, hkv, d), _rand(rng, B, N, hkv, d), _rand(rng, B, N, hq, d)
    for causal in (False, True):
        dq, dk, dv, dd = m.attn_bwd(q, k, v, do, 0.35, causal)
        o, _ = m.attn_fwd(q, k, v, 0.35, causal)
        g = hq // hkv
        for kh in range(hkv):
            heads = slice(kh * g, (kh + 1) * g)
            np.testing.assert_allclose(dv[:, :, kh].sum(axis=1), do[:, :, heads].sum(axis=(1, 2)), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dk[:, :, kh].sum(axis=1), 0.0, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dd, np.einsum("bihc,bihc->bhi", do, o), rtol=0, atol=1e-12)


def pin_decode_consistency(m):
    rng = np.random.default_rng(9)
    B, L, hq, hkv, d = 3, 12, 4, 2, 6
    kc, vc = _rand(rng, B, L, hkv, d), _rand(rng, B, L, hkv, d)
    lens = np.array([12, 1, 7])
    q = _rand(rng, B, hq, d)
    o, lse = m.attn_decode(q, kc, vc, lens, 0.4)
    for b in range(B):
        n = lens[b]
        # decode == forward with a single query row over the first n keys
        of, lf = m.attn_fwd(q[b][None, None], kc[b:b + 1, :n], vc[b:b + 1, :n], 0.4, False)
        np.testing.assert_allclose(o[b], of[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], lf[0, :, 0], rtol=0, atol=1e-13)
        # decode == last row of a causal forward whose last query is q
        qs = _rand(rng, 1, n, hq, d)
        qs[0, n - 1] = q[b]
        oc, lc = m.attn_fwd(qs, kc[b:b + 1, :n], vc[b:b + 1, :n], 0.4, True)
        np.testing.assert_allclose(o[b], oc[0, n - 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], lc[0, :, n - 1], rtol=0, atol=1e-13)


def pin_torch_sdpa(m):
    """torch's CPU attention and autograd in float64, GQA via repeat_interleave."""
    rng = np.random.default_rng(10)
    for (B, nq, nk, hq, hkv, d) in [(2, 10, 10, 4, 2, 8), (1, 7, 13, 6, 3, 5), (1, 16, 16, 2, 2, 16)]:
        q, k, v, do = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nq, hq, d)
        g = hq // hkv
        for causal in (False, True):
            tq = torch.tensor(q).transpose(1, 2).requires_grad_()
            tk = torch.tensor(k).transpose(1, 2).requires_grad_()
            tv = torch.tensor(v).transpose(1, 2).requires_grad_()
            ke, ve = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
            if causal:
                # explicit bottom-right mask (torch's is_causal aligns top-left)
                keep = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
                to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, attn_mask=keep, scale=0.45)
            else:
                to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, scale=0.45)
            to.backward(torch.tensor(do).transpose(1, 2))
            o, lse = m.attn_fwd(q, k, v, 0.45, causal)
            np.testing.assert_allclose(o, to.detach().transpose(1, 2).numpy(), rtol=0, atol=1e-12)
            s = 0.45 * torch.einsum("bhic,bhjc->bhij", tq.detach(), ke.detach())
            if causal:
                s = s.masked_fill(~keep, float("-inf"))
            np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
            dq, dk, dv, _ = m.attn_bwd(q, k, v, do, 0.45, causal)
            np.testing.assert_allclose(dq, tq.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dk, tk.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dv, tv.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)


def pin_fwd_rows(m):
    """Sampled-row forward agrees with the full forward (used for large checks)."""
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 9, 4, 3), _rand(rng, 2, 11, 2, 3), _rand(rng, 2, 11, 2, 3)
    for causal in (False, True):
        o, lse = m.attn_fwd(q, k, v, 0.9, causal)
        rows = [0, 4, 8]
        orow, lrow = m.attn_fwd_rows(q, k, v, 0.9, causal, 1, 3, rows)
        np.testing.assert_allclose(orow, o[1, rows, 3], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lrow, lse[1, 3, rows], rtol=0, atol=1e-14)


PINS = [pin_golden_fwd, pin_golden_bwd, pin_golden_decode, pin_brute_force, pin_identical_keys,
        pin_first_causal_row, pin_rows_sum_to_one, pin_shift_invariance, pin_value_tests,
        pin_finite_differences, pin_gradient_invariants, pin_decode_consistency, pin_torch_sdpa,
        pin_fwd_rows]


def pin_golden_window(m):
    data = json.load(open(GOLDEN))
    for case in data["window"]:
        q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
        o, lse = m.attn_fwd(q, k, v, _expr(case["scale"]), case["causal"], tuple(case["window"]))
        np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13, err_msg=case["name"])
        np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-13, err_msg=case["name"])


def pin_golden_varlen(m):
    data = json.load(open(GOLDEN))
    for case in data["varlen"]:
        q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
        o, lse = m.attn_fwd_varlen(q, k, v, case["cu_q"], case["cu_k"], _expr(case["scale"]), case["causal"])
        np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13, err_msg=case["name"])
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(_arr(case["lse"])))
        fin = np.isfinite(_arr(case["lse"]))
        np.testing.assert_allclose(lse[fin], _arr(case["lse"])[fin], rtol=0, atol=1e-13, err_msg=case["name"])


WINDOW_CASES = [(-1, -1), (0, 0), (1, 0), (0, 2), (3, 1), (2, -1), (-1, 2), (20, 20)]


def pin_window_brute_force(m):
    rng = np.random.default_rng(21)
    for (B, nq, nk, hq, hkv, d) in BRUTE_SHAPES:
        q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
        for window in WINDOW_CASES:
            for causal in (False, True):
                o, lse = m.attn_fwd(q, k, v, 0.6, causal, window)
                ob, lb = _brute_fwd(q, k, v, 0.6, causal, window)
                np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
                np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
                fin = np.isfinite(lb)
                np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def pin_window_special_cases(m):
    """(-1, 0) is the causal mask; a band wider than the sequence is no mask;
    (0, 0) leaves each row its own diagonal key (o = v, LSE = its score)."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 2, 9, 2, 4), _rand(rng, 2, 9, 2, 4), _rand(rng, 2, 9, 2, 4)
    oc, lc = m.attn_fwd(q, k, v, 0.5, True)
    ow, lw = m.attn_fwd(q, k, v, 0.5, False, (-1, 0))
    np.testing.assert_allclose(ow, oc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lw, lc, rtol=0, atol=1e-14)
    on, ln_ = m.attn_fwd(q, k, v, 0.5, False)
    ob, lb = m.attn_fwd(q, k, v, 0.5, False, (9, 9))
    np.testing.assert_allclose(ob, on, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lb, ln_, rtol=0, atol=1e-14)
    od, ld = m.attn_fwd(q, k, v, 0.5, False, (0, 0))
    np.testing.assert_allclose(od, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ld, 0.5 * np.einsum("bihc,bihc->bhi", q, k), rtol=0, atol=1e-13)


def pin_varlen_is_per_sequence_dense(m):
    """Each packed sequence is an independent problem: equal to a dense
    forward of that sequence alone, including Nq != Nk (bottom-right) and
    empty sequences; and equal-length packing equals the padded batch."""
    rng = np.random.default_rng(23)
    lq, lk = [3, 0, 5, 1, 4], [3, 2, 7, 1, 0]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = _rand(rng, cu_q[-1], 4, 3), _rand(rng, cu_k[-1], 2, 3), _rand(rng, cu_k[-1], 2, 3)
    for causal in (False, True):
        for window in ((-1, -1), (1, 1), (2, 0)):
            o, lse = m.attn_fwd_varlen(q, k, v, cu_q, cu_k, 0.7, causal, window)
            for b in range(len(lq)):
                a, e, c, f = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
                if e == a:
                    continue
                ob, lb = _brute_fwd(q[None, a:e], k[None, c:f], v[None, c:f], 0.7, causal, window)
                np.testing.assert_allclose(o[a:e], ob[0], rtol=0, atol=1e-12)
                np.testing.assert_array_equal(np.isneginf(lse[:, a:e]), np.isneginf(lb[0]))
    qb, kb, vb = _rand(rng, 3, 6, 2, 4), _rand(rng, 3, 6, 1, 4), _rand(rng, 3, 6, 1, 4)
    cu = np.array([0, 6, 12, 18])
    o, lse = m.attn_fwd_varlen(qb.reshape(18, 2, 4), kb.reshape(18, 1, 4), vb.reshape(18, 1, 4), cu, cu, 0.4, True)
    od, ld = m.attn_fwd(qb, kb, vb, 0.4, True)
    np.testing.assert_allclose(o, od.reshape(18, 2, 4), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, ld.transpose(1, 0, 2).reshape(2, 18), rtol=0, atol=1e-14)


def pin_golden_decode_paged(m):
    data = json.load(open(GOLDEN))
    for case in data["decode_paged"]:
        args = (_arr(case["q"]), _arr(case["k_pages"]), _arr(case["v_pages"]), np.array(case["block_table"]),
                np.array(case["cache_seqlens"]), _expr(case["scale"]))
        o, lse, kp, vp = m.attn_decode_paged(*args)
        np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13, err_msg=case["name"])
        np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-13, err_msg=case["name"])
        ap = case["append"]
        o, lse, kp, vp = m.attn_decode_paged(*args, _arr(ap["k_new"]), _arr(ap["v_new"]))
        np.testing.assert_allclose(o, _arr(ap["o"]), rtol=0, atol=1e-13, err_msg=case["name"] + " append")
        np.testing.assert_allclose(lse, _arr(ap["lse"]), rtol=0, atol=1e-13, err_msg=case["name"] + " append")
        assert vp[ap["page"], ap["row"], 0, 0] == _arr(ap["v_new"])[0, 0, 0]
        changed = np.argwhere(vp != _arr(case["v_pages"]))
        assert [tuple(x[:2]) for x in changed] == [(ap["page"], ap["row"])]


def pin_paged_decode_properties(m):
    """An identity block table is the contiguous cache; a shuffled table gives
    the same result as the rows it names; appending equals pre-writing the
    row and decoding one row longer."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, d, ps, mp = 3, 4, 2, 5, 4, 6
    lens = np.array([1, 13, 23])
    q = _rand(rng, B, Hq, d)
    kc, vc = _rand(rng, B, mp * ps, Hkv, d), _rand(rng, B, mp * ps, Hkv, d)
    ident = np.arange(B * mp).reshape(B, mp)
    kp, vp = kc.reshape(B * mp, ps, Hkv, d), vc.reshape(B * mp, ps, Hkv, d)
    o, lse, _, _ = m.attn_decode_paged(q, kp, vp, ident, lens, 0.3)
    od, ld = m.attn_decode(q, kc, vc, lens, 0.3)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-14)
    perm = rng.permutation(B * mp)
    inv = np.argsort(perm)
    table = inv[ident]  # logical page p of seq b lives at physical page inv[b*mp + p]
    o2, l2, _, _ = m.attn_decode_paged(q, kp[perm], vp[perm], table, lens, 0.3)
    np.testing.assert_allclose(o2, od, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, ld, rtol=0, atol=1e-14)
    kn, vn = _rand(rng, B, Hkv, d), _rand(rng, B, Hkv, d)
    o3, l3, kp3, vp3 = m.attn_decode_paged(q, kp[perm], vp[perm], table, lens, 0.3, kn, vn)
    kc4, vc4 = kc.copy(), vc.copy()
    for b in range(B):
        kc4[b, lens[b]], vc4[b, lens[b]] = kn[b], vn[b]
    o4, l4 = m.attn_decode(q, kc4, vc4, lens + 1, 0.3)
    np.testing.assert_allclose(o3, o4, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, l4, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(kp3[inv].reshape(B, mp * ps, Hkv, d), kc4)


def pin_golden_blocksparse(m):
    data = json.load(open(GOLDEN))
    for case in data["blocksparse"]:
        q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
        o, lse = m.attn_fwd_blocksparse(q, k, v, np.array(case["block_mask"]), case["block"], _expr(case["scale"]),
                                        case["causal"])
        np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13, err_msg=case["name"])
        want = _arr(case["lse"])
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(want))
        fin = np.isfinite(want)
        np.testing.assert_allclose(lse[fin], want[fin], rtol=0, atol=1e-13, err_msg=case["name"])


def pin_blocksparse_properties(m):
    """All-ones mask is dense attention; a block-diagonal mask is independent
    attention inside each block; a random mask equals scalar brute force with
    the block condition written out."""
    rng = np.random.default_rng(25)
    q, k, v = _rand(rng, 2, 10, 4, 3), _rand(rng, 2, 10, 2, 3), _rand(rng, 2, 10, 2, 3)
    for causal in (False, True):
        od, ld = m.attn_fwd(q, k, v, 0.8, causal)
        o1, l1 = m.attn_fwd_blocksparse(q, k, v, np.ones((4, 4)), 3, 0.8, causal)
        np.testing.assert_allclose(o1, od, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1, ld, rtol=0, atol=1e-14)
    ob, lb = m.attn_fwd_blocksparse(q, k, v, np.eye(4), 3, 0.8, False)
    for blk in range(4):
        sl = slice(3 * blk, min(3 * blk + 3, 10))
        oe, le = m.attn_fwd(q[:, sl], k[:, sl], v[:, sl], 0.8, False)
        np.testing.assert_allclose(ob[:, sl], oe, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lb[:, :, sl], le, rtol=0, atol=1e-14)
    mask = rng.integers(0, 2, (2, 4, 4, 4))
    for causal in (False, True):
        o, lse = m.attn_fwd_blocksparse(q, k, v, mask, 3, 0.8, causal)
        for b in range(2):
            for h in range(4):
                for i in range(10):
                    sc = [(j, 0.8 * float(np.dot(q[b, i, h], k[b, j, h // 2]))) for j in range(10)
                          if mask[b, h, i // 3, j // 3] and not (causal and j > i)]
                    if not sc:
                        assert np.isneginf(lse[b, h, i]) and not o[b, i, h].any()
                        continue
                    tot = sum(math.exp(x) for _, x in sc)
                    want = sum(math.exp(x) / tot * v[b, j, h // 2] for j, x in sc)
                    np.testing.assert_allclose(o[b, i, h], want, rtol=0, atol=1e-12)
                    np.testing.assert_allclose(lse[b, h, i], math.log(tot), rtol=0, atol=1e-12)


def _brute_bwd(q, k, v, do, scale, causal, window=(-1, -1)):
    """Scalar-loop gradients of sum(O * dO), the window condition written out.

    For each (batch, query head, row) the visible keys are collected with the
    same rule as the scalar forward above; p_j = exp(s_j) / sum exp(s), then
    dV_j += p_j dO_i, dp_j = dO_i . V_j, D_i = sum_j p_j dp_j,
    ds_j = p_j (dp_j - D_i), dQ_i = scale sum_j ds_j K_j, dK_j += scale ds_j Q_i.
    """
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    g = hq // hkv
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(hq):
            kh = h // g
            for i in range(nq):
                diag = i + (nk - nq)
                vis = []
                for j in range(nk):
                    if causal and j > diag:
                        continue
                    if window[0] >= 0 and j < diag - window[0]:
                        continue
                    if window[1] >= 0 and j > diag + window[1]:
                        continue
                    vis.append((j, scale * sum(q[b, i, h, c] * k[b, j, kh, c] for c in range(d))))
                if not vis:
                    continue
                top = max(sv for _, sv in vis)
                tot = sum(math.exp(sv - top) for _, sv in vis)
                pj = [(j, math.exp(sv - top) / tot) for j, sv in vis]
                dpj = {j: sum(do[b, i, h, c] * v[b, j, kh, c] for c in range(d)) for j, _ in pj}
                big_d = sum(p * dpj[j] for j, p in pj)
                for j, p in pj:
                    ds = p * (dpj[j] - big_d)
                    for c in range(d):
                        dv[b, j, kh, c] += p * do[b, i, h, c]
                        dq[b, i, h, c] += scale * ds * k[b, j, kh, c]
                        dk[b, j, kh, c] += scale * ds * q[b, i, h, c]
    return dq, dk, dv


BWD_WINDOW_CASES = [(0, 0), (1, 0), (2, -1), (-1, 2), (3, 1)]


def pin_window_bwd_brute_force(m):
    """Backward with windows (and without) against the scalar loops above, GQA
    and Nq != Nk included, causal and non-causal."""
    rng = np.random.default_rng(26)
    for (B, nq, nk, hq, hkv, d) in BRUTE_SHAPES[1:5]:
        q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
        do = _rand(rng, B, nq, hq, d)
        for window in [(-1, -1)] + BWD_WINDOW_CASES:
            for causal in (False, True):
                dq, dk, dv, _ = m.attn_bwd(q, k, v, do, 0.55, causal, window)
                bq, bk, bv = _brute_bwd(q, k, v, do, 0.55, causal, window)
                for got, want in ((dq, bq), (dk, bk), (dv, bv)):
                    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=f"{window} {causal}")


def pin_window_finite_differences(m):
    """Central differences of sum(O * dO) through the windowed forward (itself
    pinned by brute force) against the windowed backward, with GQA."""
    rng = np.random.default_rng(27)
    h = 1e-6
    for (B, nq, nk, hq, hkv, d) in [(1, 5, 5, 4, 2, 3), (1, 4, 6, 2, 1, 2)]:
        q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
        do = _rand(rng, B, nq, hq, d)
        for window in BWD_WINDOW_CASES:
            for causal in (False, True):
                grads = dict(zip("qkv", m.attn_bwd(q, k, v, do, 0.6, causal, window)[:3]))
                base = {"q": q, "k": k, "v": v}

                def loss(args):
                    return float((m.attn_fwd(args["q"], args["k"], args["v"], 0.6, causal, window)[0] * do).sum())

                for name in "qkv":
                    x = base[name]
                    num = np.zeros_like(x)
                    for idx in np.ndindex(*x.shape):
                        xp, xm = x.copy(), x.copy()
                        xp[idx] += h
                        xm[idx] -= h
                        num[idx] = (loss({**base, name: xp}) - loss({**base, name: xm})) / (2 * h)
                    err = np.abs(num - grads[name]).max() / max(1.0, np.abs(grads[name]).max())
                    assert err < 1e-6, (name, window, causal, err)


def pin_bwd_dq_rows(m):
    """Sampled-row dQ and D (used for checks too large for the full backward)
    agree with the full backward, with GQA, causal and not, and Nq != Nk
    (bottom-right causal alignment)."""
    rng = np.random.default_rng(31)
    for (B, nq, nk, hq, hkv) in [(2, 9, 9, 4, 2), (1, 6, 10, 2, 1)]:
        q, k, v = _rand(rng, B, nq, hq, 3), _rand(rng, B, nk, hkv, 3), _rand(rng, B, nk, hkv, 3)
        do = _rand(rng, B, nq, hq, 3)
        for causal in (False, True):
            dq, _, _, dd = m.attn_bwd(q, k, v, do, 0.8, causal)
            rows = [0, nq // 2, nq - 1]
            for b in range(B):
                for h in range(hq):
                    rq, rd = m.attn_bwd_dq_rows(q, k, v, do, 0.8, causal, b, h, rows)
                    np.testing.assert_allclose(rq, dq[b, rows, h], rtol=0, atol=1e-13)
                    np.testing.assert_allclose(rd, dd[b, h, rows], rtol=0, atol=1e-13)


def pin_bwd_dq_rows_finite_differences(m):
    """Central differences of sum(O * dO) with respect to the sampled query
    rows, through the forward (itself pinned by brute force), against the
    sampled-row dQ, with GQA, causal and not."""
    rng = np.random.default_rng(32)
    hstep = 1e-6
    B, nq, nk, hq, hkv, d = 1, 5, 7, 2, 1, 3
    q, k, v = _rand(rng, B, nq, hq, d), _rand(rng, B, nk, hkv, d), _rand(rng, B, nk, hkv, d)
    do = _rand(rng, B, nq, hq, d)
    rows = [0, 2, 4]
    for causal in (False, True):
        def loss(qq):
            return float((m.attn_fwd(qq, k, v, 0.7, causal)[0] * do).sum())
        for h in range(hq):
            rq, _ = m.attn_bwd_dq_rows(q, k, v, do, 0.7, causal, 0, h, rows)
            for ri, i in enumerate(rows):
                for c in range(d):
                    qp, qm = q.copy(), q.copy()
                    qp[0, i, h, c] += hstep
                    qm[0, i, h, c] -= hstep
                    num = (loss(qp) - loss(qm)) / (2 * hstep)
                    assert abs(num - rq[ri, c]) < 1e-6 * max(1.0, abs(rq[ri, c])), (causal, h, i, c, num, rq[ri, c])


PINS += [pin_bwd_dq_rows, pin_bwd_dq_rows_finite_differences]

PINS += [pin_golden_window, pin_golden_varlen, pin_window_brute_force, pin_window_special_cases,
         pin_varlen_is_per_sequence_dense, pin_golden_decode_paged, pin_paged_decode_properties,
         pin_golden_blocksparse, pin_blocksparse_properties, pin_window_bwd_brute_force,
         pin_window_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle_attention)


def test_fully_masked_row_convention():
    """Causal with Nq > Nk leaves the first rows without keys: O = 0, LSE = -inf, no NaN."""
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 5, 1, 2), _rand(rng, 1, 3, 1, 2), _rand(rng, 1, 3, 1, 2)
    o, lse = oracle.attn_fwd(q, k, v, 1.0, True)
    assert np.isneginf(lse[0, 0, :2]).all() and (o[0, :2] == 0).all()
    assert np.isfinite(lse[0, 0, 2:]).all() and not np.isnan(o).any()


def test_gqa_requires_divisibility():
    with pytest.raises(ValueError):
        oracle.attn_fwd(np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 2, 4)), np.zeros((1, 2, 2, 4)), 1.0, False)


# ------------------------------------------------------- planted mistakes --

MUTANTS = {
    "scale_dropped": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "scores_transposed": ("s = scale * (q @ k.T)", "s = scale * ((q @ k.T).T if q.shape[0] == k.shape[0] else q @ k.T)"),
    "mask_top_left": ("keep = j <= diag", "keep = j <= np.asarray(rows)[:, None]"),
    "mask_strict": ("keep = j <= diag", "keep = j < diag"),
    "gqa_modulo": ("kh = h // g\n            _, p, lse_bh", "kh = h % hkv\n            _, p, lse_bh"),
    "lse_without_max": ("m_safe[:, 0] + np.log(np.where", "np.log(np.where"),
    "lse_log2": ("m_safe[:, 0] + np.log(np.where", "m_safe[:, 0] + np.log2(np.where"),
    "no_normalise": ("e / np.where(empty, 1.0, l)", "e"),
    "dv_untransposed": ("dv[b, :, kh, :] += p.T @ doh", "dv[b, :, kh, :] += (p @ doh) if p.shape[0] == p.shape[1] else p.T @ doh"),
    "ds_sign": ("ds = p * (dp - drow)", "ds = p * (drow - dp)"),
    "ds_no_d": ("ds = p * (dp - drow)", "ds = p * dp"),
    "dq_no_scale": ("dq[b, :, h, :] = scale * (ds @ kk)", "dq[b, :, h, :] = ds @ kk"),
    "dk_overwrite_group": ("dk[b, :, kh, :] += scale", "dk[b, :, kh, :] = scale"),
    "decode_reads_whole_cache": ("kb = np.asarray(k_cache[b, :n]", "kb = np.asarray(k_cache[b, :]"),
    "decode_value_prefix_off_by_one": ("vb = np.asarray(v_cache[b, :n]", "vb = np.asarray(v_cache[b, 1:n + 1]"),
    "window_left_strict": ("j >= diag - wl", "j > diag - wl"),
    "window_sides_swapped": ("j >= diag - wl, s", "j >= diag - wr, s"),
    "window_top_left": ("diag = np.asarray(rows)[:, None] + (nk - nq)", "diag = np.asarray(rows)[:, None] + 0 * (nk - nq)"),
    "varlen_keys_from_query_offsets": ("k[None, k0:k1], v[None, k0:k1]", "k[None, q0:q0 + (k1 - k0)], v[None, q0:q0 + (k1 - k0)]"),
    "paged_row_within_page": ("return pages[np.asarray(block_table)[b, t // page_size], t % page_size]",
                              "return pages[np.asarray(block_table)[b, t // page_size], (t + 1) % page_size]"),
    "paged_append_before_last_row": ("            t = int(lens[b])\n", "            t = int(lens[b]) - 1\n"),
    "paged_append_not_attended": ("        lens = lens + 1\n", "        lens = lens + 0\n"),
    "blocksparse_mask_transposed": ("return bm[np.arange(nq)[:, None] // block, np.arange(nk)[None, :] // block]",
                                    "return bm.T[np.arange(nq)[:, None] // block, np.arange(nk)[None, :] // block]"),
    "blocksparse_block_off_by_one": ("bm[np.arange(nq)[:, None] // block, np.arange(nk)[None, :] // block]",
                                     "bm[np.arange(nq)[:, None] // block, np.minimum(np.arange(nk)[None, :] + 1, nk - 1) // block]"),
    "blocksparse_mask_ignored": ("        s = np.where(keep_extra, s, -np.inf)", "        s = s"),
    "bwd_window_dropped": ("_, p, _ = head_probs(qh, kk, scale, causal, window=window)",
                           "_, p, _ = head_probs(qh, kk, scale, causal)"),
    "bwd_window_left_only": ("_, p, _ = head_probs(qh, kk, scale, causal, window=window)",
                             "_, p, _ = head_probs(qh, kk, scale, causal, window=(window[0], -1))"),
    "dq_rows_d_dropped": ("dsr = pr * (dpr - dr[:, None])", "dsr = pr * dpr"),
    "dq_rows_wrong_kv_head": ("kv_head = h // _check_heads(hq, hkv)", "kv_head = h % hkv"),
    "dq_rows_top_left_mask": ("head_probs(qr, kk, scale, causal, rows=rows, nq=q.shape[1])",
                              "head_probs(qr, kk, scale, causal, rows=rows, nq=k.shape[1])"),
    "varlen_lse_row_major": ("lse[:, q0:q1] = lb[0]", "lse[:, q0:q1] = lb[0][::-1] if lb.shape[1] > 1 else lb[0]"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(oracle_attention.__file__).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
