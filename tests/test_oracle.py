"""Pins for the fp64 oracle. Each check rests on something other than the oracle itself.

* a hand-worked closed-form example (tests/golden/hand_worked_s3.json);
* brute force: pure-Python loops with math.fsum on tiny inputs;
* closed forms: Q = 0, S = 1, constant V, causal row 0 and each segment's first row;
* invariants: key shift, packed = per-segment runs, GQA = MHA with repeated K/V,
  head-share slice, causal last row = non-causal last row;
* torch's CPU scaled_dot_product_attention in float64 (forward and autograd backward);
* central finite differences of <O, dO> for the backward, plus sum(dK) = 0 and
  sum(dV) = sum(dO) per kv head and segment.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from seeded_inputs import cu_seqlens_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _mask_kinds():
    # (causal, lengths or None)
    return [(False, None), (True, None), (True, [3, 5, 1, 7]), (False, [6, 10])]


# ---------------------------------------------------------------- golden -----

def _ev(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "log": math.log, "exp": math.exp})


@pytest.mark.parametrize("kind", ["causal", "noncausal"])
def test_hand_worked_example(kind):
    with open(os.path.join(GOLDEN, "hand_worked_s3.json"), encoding="utf-8") as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.array(g["k"], dtype=np.float64)[None, :, None, :]
    v = np.array(g["v"], dtype=np.float64)[None, :, None, :]
    o, lse = oracle.attention_fwd(q, k, v, causal=(kind == "causal"), scale=g["scale"])
    want_o = np.array([[_ev(x) for x in row] for row in g[kind]["o"]])
    want_l = np.array([_ev(x) for x in g[kind]["lse"]])
    np.testing.assert_allclose(o[0, :, 0, :], want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], want_l, rtol=0, atol=1e-14)
    o2, l2 = oracle.attention_fwd_rows(q, k, v, [(0, 0, i) for i in range(3)], causal=(kind == "causal"),
                                       scale=g["scale"])
    np.testing.assert_allclose(o2, want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, want_l, rtol=0, atol=1e-14)


# ------------------------------------------------------------ brute force ----

def _brute_fwd(q, k, v, causal, scale, lengths):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    seg = [0] * S
    if lengths is not None:
        pos = 0
        for n, L in enumerate(lengths):
            for t in range(L):
                seg[pos + t] = n
            pos += L
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                keys = [j for j in range(S) if seg[j] == seg[i] and (not causal or j <= i)]
                s = [scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, h // G, d]) for d in range(D))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                lse[b, h, i] = mx + math.log(tot)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(wj * float(v[b, j, h // G, d]) for wj, j in zip(w, keys)) / tot
    return o, lse


@pytest.mark.parametrize("causal,lengths", _mask_kinds())
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2)])
def test_forward_matches_brute_force(causal, lengths, hq, hkv):
    S = 16
    D = 5
    B = 1 if lengths is not None else 2
    q = _rand((B, S, hq, D), 1)
    k = _rand((B, S, hkv, D), 2)
    v = _rand((B, S, hkv, D), 3)
    scale = 0.37
    cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu)
    bo, bl = _brute_fwd(q, k, v, causal, scale, lengths)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-13)
    picks = [(b, h, i) for b in range(B) for h in range(hq) for i in range(S)]
    ro, rl = oracle.attention_fwd_rows(q, k, v, picks, causal=causal, scale=scale, cu_seqlens=cu)
    np.testing.assert_allclose(ro, np.array([bo[b, i, h] for b, h, i in picks]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(rl, np.array([bl[b, h, i] for b, h, i in picks]), rtol=0, atol=1e-13)


def test_forward_brute_force_multiple_row_blocks(monkeypatch):
    # more rows than one oracle row block, so the block split is exercised
    monkeypatch.setattr(oracle.attention, "ROW_BLOCK", 7)
    S, D = 23, 3
    q, k, v = _rand((1, S, 2, D), 4), _rand((1, S, 1, D), 5), _rand((1, S, 1, D), 6)
    for causal, lengths in [(True, None), (True, [9, 14]), (False, [5, 18])]:
        cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
        o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=0.5, cu_seqlens=cu, workers=3)
        bo, bl = _brute_fwd(q, k, v, causal, 0.5, lengths)
        np.testing.assert_allclose(o, bo, atol=1e-13)
        np.testing.assert_allclose(lse, bl, atol=1e-13)


# ------------------------------------------------------------ closed forms ---

@pytest.mark.parametrize("causal,lengths", _mask_kinds())
def test_zero_queries_give_mean_of_visible_values(causal, lengths):
    S, D = 16, 4
    q = np.zeros((1, S, 2, D))
    k = _rand((1, S, 1, D), 7)
    v = _rand((1, S, 1, D), 8)
    cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=0.3, cu_seqlens=cu)
    start, end = oracle.segment_bounds(S, cu)
    for i in range(S):
        lo, hi = int(start[i]), (i + 1 if causal else int(end[i]))
        for h in range(2):
            np.testing.assert_allclose(o[0, i, h], v[0, lo:hi, 0].mean(axis=0), atol=1e-14)
            assert abs(lse[0, h, i] - math.log(hi - lo)) < 1e-14


def test_single_token():
    q, k, v = _rand((3, 1, 4, 8), 9), _rand((3, 1, 2, 8), 10), _rand((3, 1, 2, 8), 11)
    for causal in (True, False):
        o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=0.25)
        for h in range(4):
            np.testing.assert_allclose(o[:, 0, h], v[:, 0, h // 2], atol=1e-15)
            np.testing.assert_allclose(lse[:, h, 0], 0.25 * np.sum(q[:, 0, h] * k[:, 0, h // 2], axis=-1),
                                       atol=1e-14)


def test_one_token_segments_backward():
    # each row sees only its own key: P = 1, so dS = P (dP - Delta) = dO.V - dO.V = 0,
    # dQ = dK = 0, and dV of a key is the sum of dO over the query heads of its group
    S, D = 6, 5
    q, k, v, do = _rand((1, S, 4, D), 40), _rand((1, S, 2, D), 41), _rand((1, S, 2, D), 42), _rand((1, S, 4, D), 43)
    cu = cu_seqlens_from_lengths([1] * S)
    for causal in (True, False):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=0.7, cu_seqlens=cu)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)
        np.testing.assert_allclose(dk, 0.0, atol=1e-14)
        np.testing.assert_allclose(dv, do.reshape(1, S, 2, 2, D).sum(axis=3), atol=1e-14)


def test_constant_values_give_that_row():
    S, D = 20, 6
    q, k = _rand((1, S, 2, D), 12, 3.0), _rand((1, S, 2, D), 13, 3.0)
    row = _rand((D,), 14)
    v = np.broadcast_to(row, (1, S, 2, D)).copy()
    for causal, lengths in _mask_kinds():
        if lengths is not None and sum(lengths) != S:
            lengths = [4, 16]
        cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
        o, _ = oracle.attention_fwd(q, k, v, causal=causal, scale=0.9, cu_seqlens=cu)
        np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), atol=1e-13)


def test_first_row_of_each_causal_segment_copies_value():
    lengths = [5, 9, 2]
    S, D = sum(lengths), 4
    q, k, v = _rand((1, S, 2, D), 15), _rand((1, S, 2, D), 16), _rand((1, S, 2, D), 17)
    cu = cu_seqlens_from_lengths(lengths)
    o, lse = oracle.attention_fwd(q, k, v, causal=True, scale=0.6, cu_seqlens=cu)
    for s0 in cu[:-1]:
        np.testing.assert_allclose(o[0, s0], v[0, s0], atol=1e-15)
        np.testing.assert_allclose(lse[0, :, s0], 0.6 * np.sum(q[0, s0] * k[0, s0], axis=-1), atol=1e-14)


def test_probabilities_sum_to_one():
    # the row sums of P are what the LSE normalises: sum_j exp(s_ij - LSE_i) = 1
    S, D = 33, 8
    q, k, v = _rand((1, S, 1, D), 18, 2.0), _rand((1, S, 1, D), 19, 2.0), _rand((1, S, 1, D), 20)
    _, lse = oracle.attention_fwd(q, k, v, causal=True, scale=0.5)
    for i in range(S):
        s = 0.5 * (k[0, :i + 1, 0] @ q[0, i, 0])
        assert abs(np.sum(np.exp(s - lse[0, 0, i])) - 1.0) < 1e-12


# -------------------------------------------------------------- invariants ---

def test_causal_last_row_equals_noncausal_last_row():
    q, k, v = _rand((2, 40, 3, 8), 21), _rand((2, 40, 3, 8), 22), _rand((2, 40, 3, 8), 23)
    oc, lc = oracle.attention_fwd(q, k, v, causal=True, scale=0.4)
    on, ln = oracle.attention_fwd(q, k, v, causal=False, scale=0.4)
    np.testing.assert_allclose(oc[:, -1], on[:, -1], atol=1e-14)
    np.testing.assert_allclose(lc[:, :, -1], ln[:, :, -1], atol=1e-14)
    assert not np.allclose(oc[:, 0], on[:, 0])


@pytest.mark.parametrize("causal", [True, False])
def test_key_shift_invariance(causal):
    S, D = 24, 8
    q, k, v = _rand((1, S, 2, D), 24), _rand((1, S, 1, D), 25), _rand((1, S, 1, D), 26)
    u = _rand((D,), 27)
    o1, l1 = oracle.attention_fwd(q, k, v, causal=causal, scale=0.7)
    o2, l2 = oracle.attention_fwd(q, k + u, v, causal=causal, scale=0.7)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.7 * np.einsum("bshd,d->bhs", q, u), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_packed_equals_per_segment_runs(causal):
    lengths = [7, 1, 12, 4]
    S, D = sum(lengths), 6
    q, k, v = _rand((1, S, 4, D), 28), _rand((1, S, 2, D), 29), _rand((1, S, 2, D), 30)
    do = _rand((1, S, 4, D), 31)
    cu = cu_seqlens_from_lengths(lengths)
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=0.5, cu_seqlens=cu)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=0.5, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        so, sl = oracle.attention_fwd(q[:, a:b], k[:, a:b], v[:, a:b], causal=causal, scale=0.5)
        np.testing.assert_allclose(o[:, a:b], so, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, a:b], sl, atol=1e-14)
        gq, gk, gv = oracle.attention_bwd(q[:, a:b], k[:, a:b], v[:, a:b], do[:, a:b], causal=causal, scale=0.5)
        np.testing.assert_allclose(dq[:, a:b], gq, atol=1e-13)
        np.testing.assert_allclose(dk[:, a:b], gk, atol=1e-13)
        np.testing.assert_allclose(dv[:, a:b], gv, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    S, D, Hq, Hkv = 19, 8, 6, 2
    G = Hq // Hkv
    q, k, v, do = (_rand((2, S, Hq, D), 32), _rand((2, S, Hkv, D), 33), _rand((2, S, Hkv, D), 34),
                   _rand((2, S, Hq, D), 35))
    kr = np.repeat(k, G, axis=2)
    vr = np.repeat(v, G, axis=2)
    o, l_ = oracle.attention_fwd(q, k, v, causal=True, scale=0.3)
    orr, lr = oracle.attention_fwd(q, kr, vr, causal=True, scale=0.3)
    np.testing.assert_allclose(o, orr, atol=1e-14)
    np.testing.assert_allclose(l_, lr, atol=1e-14)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.3)
    dqr, dkr, dvr = oracle.attention_bwd(q, kr, vr, do, causal=True, scale=0.3)
    np.testing.assert_allclose(dq, dqr, atol=1e-13)
    np.testing.assert_allclose(dk, dkr.reshape(2, S, Hkv, G, D).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dvr.reshape(2, S, Hkv, G, D).sum(axis=3), atol=1e-13)


def test_head_share_slice_equals_full_run():
    # one GPU's Ulysses share (half the heads, full sequence) is the matching slice of the full result
    S, D, Hq, Hkv = 21, 4, 8, 2
    q, k, v = _rand((1, S, Hq, D), 36), _rand((1, S, Hkv, D), 37), _rand((1, S, Hkv, D), 38)
    o, l_ = oracle.attention_fwd(q, k, v, causal=True, scale=0.5)
    half_q, half_kv = Hq // 2, Hkv // 2
    so, sl = oracle.attention_fwd(q[:, :, half_q:], k[:, :, half_kv:], v[:, :, half_kv:], causal=True, scale=0.5)
    np.testing.assert_allclose(so, o[:, :, half_q:], atol=1e-15)
    np.testing.assert_allclose(sl, l_[:, half_q:], atol=1e-15)


# ------------------------------------------------------------------- torch ---

def _torch_ref(q, k, v, do, causal, scale, lengths):
    torch = pytest.importorskip("torch")
    tq = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    G = q.shape[2] // k.shape[2]
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    S = q.shape[1]
    mask = None
    if lengths is not None:
        seg = torch.repeat_interleave(torch.arange(len(lengths)), torch.tensor(lengths))
        mask = seg[:, None] == seg[None, :]
        if causal:
            mask = mask & torch.ones(S, S, dtype=torch.bool).tril()
        o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask, scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do).permute(0, 2, 1, 3))
    back = lambda t: t.detach().permute(0, 2, 1, 3).numpy()
    return back(o), back(tq.grad), back(tk.grad), back(tv.grad)


@pytest.mark.parametrize("causal,lengths", _mask_kinds())
def test_matches_torch_sdpa_fp64(causal, lengths):
    S = 16 if lengths is not None else 64
    D, Hq, Hkv = 16, 4, 2
    q, k, v, do = (_rand((1, S, Hq, D), 40), _rand((1, S, Hkv, D), 41), _rand((1, S, Hkv, D), 42),
                   _rand((1, S, Hq, D), 43))
    cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
    to, tdq, tdk, tdv = _torch_ref(q, k, v, do, causal, 0.25, lengths)
    o, _ = oracle.attention_fwd(q, k, v, causal=causal, scale=0.25, cu_seqlens=cu)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=0.25, cu_seqlens=cu)
    np.testing.assert_allclose(o, to, atol=1e-12)
    np.testing.assert_allclose(dq, tdq, atol=1e-12)
    np.testing.assert_allclose(dk, tdk, atol=1e-12)
    np.testing.assert_allclose(dv, tdv, atol=1e-12)


# ------------------------------------------------------- backward pins ------

def _loss(q, k, v, do, causal, scale, cu):
    o, _ = oracle.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal,lengths", [(True, None), (False, None), (True, [5, 9, 4])])
def test_backward_matches_finite_differences(causal, lengths):
    S, D, Hq, Hkv = 18, 4, 4, 2
    q, k, v, do = (_rand((1, S, Hq, D), 50), _rand((1, S, Hkv, D), 51), _rand((1, S, Hkv, D), 52),
                   _rand((1, S, Hq, D), 53))
    cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
    scale = 0.45
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=scale, cu_seqlens=cu)
    rng = np.random.default_rng(54)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(64):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, causal, scale, cu)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, causal, scale, cu)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal,lengths", [(True, None), (False, None), (True, [6, 3, 11])])
def test_gradient_sums(causal, lengths):
    # sum_j dK_j = 0 (the softmax is invariant to a common key shift) and
    # sum_j dV_j = sum_i dO_i (each row of P sums to one), per kv head and segment
    S, D, Hq, Hkv = 20, 8, 6, 2
    G = Hq // Hkv
    q, k, v, do = (_rand((1, S, Hq, D), 60), _rand((1, S, Hkv, D), 61), _rand((1, S, Hkv, D), 62),
                   _rand((1, S, Hq, D), 63))
    cu = cu_seqlens_from_lengths(lengths if lengths is not None else [S])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=0.5,
                                      cu_seqlens=None if lengths is None else cu)
    for a, b in zip(cu[:-1], cu[1:]):
        for kv in range(Hkv):
            np.testing.assert_allclose(dk[0, a:b, kv].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[0, a:b, kv].sum(axis=0),
                                       do[0, a:b, kv * G:(kv + 1) * G].sum(axis=(0, 1)), atol=1e-12)


@pytest.mark.parametrize("lengths", [None, [9, 20, 11]])
def test_group_backward_and_row_dq_match_full_backward(lengths, monkeypatch):
    monkeypatch.setattr(oracle.attention, "ROW_BLOCK", 8)
    S, D, Hq, Hkv = 40, 8, 6, 2
    G = Hq // Hkv
    q, k, v, do = (_rand((1, S, Hq, D), 70), _rand((1, S, Hkv, D), 71), _rand((1, S, Hkv, D), 72),
                   _rand((1, S, Hq, D), 73))
    cu = None if lengths is None else cu_seqlens_from_lengths(lengths)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.3, cu_seqlens=cu, workers=2)
    gq, gk, gv = oracle.attention_bwd_group(q, k, v, do, b=0, kv_head=1, causal=True, scale=0.3,
                                            cu_seqlens=cu, workers=3)
    np.testing.assert_allclose(gq, dq[0, :, G:2 * G], atol=1e-13)
    np.testing.assert_allclose(gk, dk[0, :, 1], atol=1e-13)
    np.testing.assert_allclose(gv, dv[0, :, 1], atol=1e-13)
    picks = [(0, h, i) for h in (0, 5) for i in (0, 1, 17, 39)]
    rq = oracle.attention_dq_rows(q, k, v, do, picks, causal=True, scale=0.3, cu_seqlens=cu)
    np.testing.assert_allclose(rq, np.array([dq[0, i, h] for _, h, i in picks]), atol=1e-13)


@pytest.mark.parametrize("causal,lengths", [(True, None), (False, None), (True, [9, 20, 11]), (False, [9, 20, 11])])
def test_key_row_dkdv_match_full_backward(causal, lengths):
    S, D, Hq, Hkv = 40, 8, 6, 2
    q, k, v, do = (_rand((2, S, Hq, D), 80), _rand((2, S, Hkv, D), 81), _rand((2, S, Hkv, D), 82),
                   _rand((2, S, Hq, D), 83))
    cu = None
    if lengths is not None:
        q, k, v, do = q[:1], k[:1], v[:1], do[:1]
        cu = cu_seqlens_from_lengths(lengths)
    _, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=0.3, cu_seqlens=cu, workers=2)
    picks = [(b, kv, j) for b in range(q.shape[0]) for kv in range(Hkv) for j in (0, 1, 8, 9, 28, 39)]
    rk, rv = oracle.attention_dkdv_rows(q, k, v, do, picks, causal=causal, scale=0.3, cu_seqlens=cu, workers=2)
    np.testing.assert_allclose(rk, np.array([dk[b, j, kv] for b, kv, j in picks]), atol=1e-13)
    np.testing.assert_allclose(rv, np.array([dv[b, j, kv] for b, kv, j in picks]), atol=1e-13)


# ------------------------------------------------------------------- fp8 -----

def test_e4m3_decoder_matches_torch_for_all_codes():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert ours[1] == 2.0 ** -9  # smallest subnormal


# ----------------------------------------------------------- merging -----

@pytest.mark.parametrize("nchunk,hq,hkv", [(2, 1, 1), (3, 2, 1), (4, 4, 2)])
def test_merge_of_key_chunks_equals_full_attention(nchunk, hq, hkv):
    # non-causal attention over all keys = merge of attention over each key chunk
    S, D = 8, 5
    q, k, v = _rand((1, S, hq, D), 50), _rand((1, S, hkv, D), 51), _rand((1, S, hkv, D), 52)
    ro, rl = oracle.attention_fwd(q, k, v, causal=False, scale=0.4)
    bounds = np.linspace(0, S, nchunk + 1).astype(int)
    o, l_ = None, None
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        # attention of every query over the keys c0 .. c1-1 only, written out here
        po = np.zeros_like(q); pl = np.zeros((1, hq, S))
        for h in range(hq):
            kv = h // (hq // hkv)
            s = 0.4 * q[0, :, h] @ k[0, c0:c1, kv].T
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            po[0, :, h] = (w / w.sum(axis=1, keepdims=True)) @ v[0, c0:c1, kv]
            pl[0, h] = m[:, 0] + np.log(w.sum(axis=1))
        o, l_ = (po, pl) if o is None else oracle.merge_partials(o, l_, po, pl)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nchunk", [2, 4])
def test_ring_layout_causal(nchunk):
    # query chunk r: non-causal against key chunks c < r, causal against c = r,
    # merged in ring order = rows of chunk r of the full causal attention
    S, D, H = 12, 4, 2
    q, k, v = _rand((1, S, H, D), 60), _rand((1, S, H, D), 61), _rand((1, S, H, D), 62)
    ro, rl = oracle.attention_fwd(q, k, v, causal=True, scale=0.5)
    L = S // nchunk
    for r in range(nchunk):
        qs = slice(r * L, (r + 1) * L)
        o, l_ = None, None
        for c in range(r + 1):
            ks = slice(c * L, (c + 1) * L)
            po, pl = oracle.attention_fwd(q[:, qs], k[:, ks], v[:, ks], causal=(c == r), scale=0.5)
            o, l_ = (po, pl) if o is None else oracle.merge_partials(o, l_, po, pl)
        np.testing.assert_allclose(o, ro[:, qs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_, rl[:, :, qs], rtol=0, atol=1e-12)


def test_merge_with_empty_part_and_commutes():
    o1, l1 = _rand((2, 5, 3, 4), 70), _rand((2, 3, 5), 71)
    o2, l2 = _rand((2, 5, 3, 4), 72), _rand((2, 3, 5), 73)
    empty_l = np.full_like(l1, -np.inf)
    o, l_ = oracle.merge_partials(o1, l1, np.zeros_like(o1), empty_l)
    np.testing.assert_array_equal(l_, l1)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    o, l_ = oracle.merge_partials(np.zeros_like(o1), empty_l, np.zeros_like(o1), empty_l)
    assert np.all(np.isneginf(l_)) and np.all(o == 0)
    oa, la = oracle.merge_partials(o1, l1, o2, l2)
    ob, lb = oracle.merge_partials(o2, l2, o1, l1)
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-14)


def test_merge_brute_force_two_rows():
    # LSE = log(e^a + e^b) and O = (e^a x + e^b y) / (e^a + e^b), by math.fsum on scalars
    rng = np.random.default_rng(80)
    for _ in range(20):
        a, b = rng.uniform(-30, 30, 2)
        x, y = rng.standard_normal(2)
        o, l_ = oracle.merge_partials(np.full((1, 1, 1, 1), x), np.full((1, 1, 1), a),
                                      np.full((1, 1, 1, 1), y), np.full((1, 1, 1), b))
        ea, eb = math.exp(a), math.exp(b)
        assert abs(l_[0, 0, 0] - math.log(math.fsum([ea, eb]))) <= 1e-12 * max(1.0, abs(a), abs(b))
        assert abs(o[0, 0, 0, 0] - math.fsum([ea * x, eb * y]) / math.fsum([ea, eb])) <= 1e-12
