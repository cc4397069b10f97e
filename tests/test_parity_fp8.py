"""GPU parity of the FP8 E4M3 forward (through the C ABI) against the fp64 oracle.

The oracle runs on the dequantised inputs (its own E4M3 decoder times the
per-tensor fp32 descale), so the comparison measures the kernel, not the input
quantisation. Tolerances: O rel-L2 <= 5e-2 (the fp8 output bound) and LSE
max-abs <= 1e-3 (the scores are exact products of E4M3 values accumulated in
fp32, so the LSE keeps the bf16 path's bound).
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import TOL_FP8_REL, TOL_LSE, dev_i32, dev_u8, host, max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _run_fp8(B, Hq, Hkv, S, D, causal, lengths=None, seed=21, qk_std=1.0, split=True):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"fp8 case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} seed={seed} "
          f"qk_std={qk_std} split={split}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, fp8=True, with_do=False, qk_std=qk_std)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu, scale=scale, split=split)
    torch.cuda.synchronize()
    qv = oracle.e4m3_decode(x.q_bits) * float(x.descale[0])
    kv = oracle.e4m3_decode(x.k_bits) * float(x.descale[1])
    vv = oracle.e4m3_decode(x.v_bits) * float(x.descale[2])
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    o_h, l_h = host(o), host(lse)
    rr, rlse = rel_l2(o_h, ro), max_abs(l_h, rl)
    msg = f"fp8 O relL2={rr:.3e} LSE maxabs={rlse:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(l_h)), msg
    assert rr <= TOL_FP8_REL and rlse <= TOL_LSE, msg
    return o, lse


CASES = [
    # B, Hq, Hkv, S, D, causal, lengths
    (1, 2, 2, 256, 128, True, None),
    (1, 2, 2, 256, 128, False, None),
    (1, 1, 1, 1, 128, True, None),
    (2, 3, 1, 77, 128, True, None),
    (2, 4, 2, 333, 128, False, None),
    (1, 8, 1, 1000, 128, True, None),
    (1, 4, 1, 700, 128, True, [300, 400]),
    (1, 2, 2, 700, 128, False, [1, 299, 400]),
    (1, 8, 1, 4096, 128, True, None),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", CASES)
def test_fp8_forward(B, Hq, Hkv, S, D, causal, lengths):
    _run_fp8(B, Hq, Hkv, S, D, causal, lengths=lengths)


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [(1, 4, 2, 1000, True, None), (2, 3, 1, 333, False, None),
                                                       (1, 2, 2, 700, True, [100, 37, 563])])
def test_fp8_forward_block_geometries(B, Hq, Hkv, S, causal, lengths, monkeypatch):
    """Both fp8 forward geometries (ATTN_FWD_WAVES=4: 128-query blocks, 8: 256-query blocks) meet the oracle
    bar and give bitwise the same O and LSE."""
    import torch
    outs = []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        outs.append(_run_fp8(B, Hq, Hkv, S, 128, causal, lengths=lengths, seed=23, split=False))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def _rising_fp8(B, Hq, Hkv, S, seed, rise_log2=150.0):
    """E4M3 inputs (per-tensor scales) of N(0,1) values with channel 0 of Q set to 16 and channel 0 of K rising
    along the sequence, so that a row's scores grow by up to `rise_log2` (log2 units) past its first keys."""
    D = 128
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, with_do=False)
    c = 1.0 / np.sqrt(D) * np.log2(np.e)
    q, k, v = (si.bf16_bits_to_f64(b).astype(np.float32) for b in (x.q_bits, x.k_bits, x.v_bits))
    q[..., 0] = 16.0
    k[..., 0] = np.arange(S)[None, :, None] * (rise_log2 / (16.0 * c * S))
    return [si.e4m3_quantize(t) for t in (q, k, v)]


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,ks_ok", [(1, 4, 2, 1536, True, False), (1, 2, 1, 1200, False, False),
                                                     (1, 1, 1, 8192, True, True)])
def test_fp8_rising_scores_redo_with_the_tracked_maximum(B, Hq, Hkv, S, causal, ks_ok, monkeypatch):
    """Scores rising by up to 150 (log2 units) along each row: past the first tile's maximum plus its margin a
    probability leaves the E4M3 range, becomes NaN in O's accumulator, and the wave redoes its rows with the
    tracked maximum. Both block geometries (and, for the last shape, the key split) meet the fp8 O bar, and the
    two geometries agree bitwise. The LSE bound grows with the size of the dot products: the E4M3 MFMA does
    not add its 64 products exactly but drops low-order bits against the largest (measured on MI355X: up to
    2^-12.2 of the sum of |products|), which at scores near 100 moves the LSE by ~1e-2; the bound is
    1e-3 + 2^-11 scale max_j sum_d |q_id k_jd| per row."""
    import torch
    import long_context_exact_fwd_amd as lca
    D = 128
    print(f"fp8 rising scores B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal}", flush=True)
    (q8h, dq), (k8h, dk), (v8h, dv) = _rising_fp8(B, Hq, Hkv, S, 61)
    q8, k8, v8 = dev_u8(q8h), dev_u8(k8h), dev_u8(v8h)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in (dq, dk, dv)]
    scale = 1.0 / np.sqrt(D)
    qv = oracle.e4m3_decode(q8h) * float(dq)
    kv = oracle.e4m3_decode(k8h) * float(dk)
    vv = oracle.e4m3_decode(v8h) * float(dv)
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    G = Hq // Hkv
    lse_bound = np.empty_like(rl)
    for h in range(Hq):
        dots = np.abs(qv[0, :, h]) @ np.abs(kv[0, :, h // G]).T
        if causal:
            dots = np.tril(dots)
        lse_bound[0, h] = TOL_LSE + 2.0 ** -11 * scale * dots.max(axis=1)
    outs = []
    runs = [("4", False), ("8", False)] + ([("4", True)] if ks_ok else [])
    for waves, split in runs:
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, scale=scale, split=split)
        torch.cuda.synchronize()
        o_h, l_h = host(o), host(lse)
        rr, rlse = rel_l2(o_h, ro), max_abs(l_h, rl)
        worst = float(np.max(np.abs(l_h - rl) / lse_bound))
        print(f"waves={waves} split={split}: O relL2={rr:.3e} LSE maxabs={rlse:.3e} ({worst:.2f} of its bound)",
              flush=True)
        assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(l_h))
        assert rr <= TOL_FP8_REL and worst <= 1.0
        if not split:
            outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # the ring-merge forward redoes the same waves: into an empty running result it gives the forward's O, LSE
    o_acc = torch.empty((B, S, Hq, D), dtype=torch.float32, device="cuda")
    l_acc = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, l_acc, causal=causal, accumulate=False, scale=scale)
    torch.cuda.synchronize()
    o_h, l_h = host(o_acc), host(l_acc)
    rr = rel_l2(o_h, ro)
    worst = float(np.max(np.abs(l_h - rl) / lse_bound))
    print(f"fwd_fp8_merge: O relL2={rr:.3e} LSE {worst:.2f} of its bound", flush=True)
    assert np.all(np.isfinite(o_h)) and rr <= TOL_FP8_REL and worst <= 1.0


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths,ks", [(1, 1, 1, 8192, True, None, 4),
                                                          (1, 2, 1, 8192, False, [3000, 5192], 4),
                                                          (1, 8, 1, 4096, True, None, 2)])
def test_fp8_forward_key_split(B, Hq, Hkv, S, causal, lengths, ks):
    """Small grids split the key tiles over ks workgroups (shares combined by the same kernel as the bf16
    path); both the split and the unsplit fp8 forward meet the fp8 bar."""
    import long_context_exact_fwd_amd as lca
    assert lca.fwd_workspace_bytes(B, Hq, Hkv, S, 128) == -(-4 * ks * B * S * Hq * 128 // 256) * 256 + 4 * ks * B * Hq * S
    for split in (True, False):
        _run_fp8(B, Hq, Hkv, S, 128, causal, lengths=lengths, seed=22, split=split)


def test_fp8_peaky_scores_exercise_rescaling():
    """Q and K scaled by 3: the running maximum moves often, so the 0.5 (log2) rescale path runs."""
    _run_fp8(1, 4, 1, 1500, 128, True, seed=22, qk_std=3.0)


BWD_CASES = [
    # B, Hq, Hkv, S, causal, lengths
    (1, 2, 2, 256, True, None),
    (2, 3, 1, 77, False, None),
    (1, 8, 1, 1000, True, None),
    (1, 4, 1, 700, True, [300, 1, 399]),
    (1, 14, 2, 2048, True, None),
]


def _fp8_bwd_case(B, Hq, Hkv, S, causal, lengths, exact_o):
    import torch
    import long_context_exact_fwd_amd as lca
    from tests.gpu_helpers import TOL_GRAD_REL, check_grads
    D = 128
    print(f"fp8 bwd case B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths} exact_o={exact_o}",
          flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 23, lengths=lengths, fp8=True, with_do=True)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    do = lca.bf16_from_bits(x.do_bits, "cuda")
    scale = 1.0 / np.sqrt(D)
    qv = oracle.e4m3_decode(x.q_bits) * float(x.descale[0])
    kv = oracle.e4m3_decode(x.k_bits) * float(x.descale[1])
    vv = oracle.e4m3_decode(x.v_bits) * float(x.descale[2])
    if exact_o:
        ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
        o = torch.from_numpy(ro).to(torch.bfloat16).cuda()
        lse = torch.from_numpy(rl).to(torch.float32).cuda()
    else:
        o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu, scale=scale)
    dq, dk, dv = lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, x.values("do"), causal=causal, scale=scale,
                                      cu_seqlens=x.cu_seqlens, workers=None)
    if exact_o:
        check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)], tag="fp8 bwd")
    else:
        errs = [rel_l2(host(g), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
        print(f"fp8 fwd+bwd: dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
        assert max(errs) <= TOL_FP8_REL


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", BWD_CASES)
def test_fp8_backward(B, Hq, Hkv, S, causal, lengths):
    """attn_bwd_fp8 against the oracle's backward on the dequantised inputs, given the exact O (bf16) and
    LSE: the exact gradient, so the bf16 gradient bound applies, rel-L2 <= 1e-2 per tensor."""
    _fp8_bwd_case(B, Hq, Hkv, S, causal, lengths, exact_o=True)


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [BWD_CASES[2], BWD_CASES[3]])
def test_fp8_forward_then_backward(B, Hq, Hkv, S, causal, lengths):
    """attn_fwd_fp8 then attn_bwd_fp8 on its own O and LSE: the forward's fp8 probabilities enter the
    gradient through Delta = rowsum(dO * O), so the fp8 bound applies, rel-L2 <= 5e-2 per tensor."""
    _fp8_bwd_case(B, Hq, Hkv, S, causal, lengths, exact_o=False)


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [(1, 2, 1, 2, True, None), (2, 4, 2, 9, True, None),
                                                       (1, 4, 2, 33, False, None),
                                                       (1, 4, 1, 128, True, [1, 2, 7, 50, 68])])
def test_fp8_few_key_rows_backward_against_the_exact_gradient(B, Hq, Hkv, S, causal, lengths):
    """attn_bwd_fp8 on rows that see fewer than 64 keys, given the exact O (bf16) and LSE: Delta comes from
    its definition there (the widened codes are exact, so P and dP are those of the dequantised inputs),
    and the gradients are held to rel-L2 <= 5e-3 of the exact ones, half the general bar, on three seeds."""
    import torch
    import long_context_exact_fwd_amd as lca
    D = 128
    for seed in (91, 92, 93):
        tag = f"fp8 few keys B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths} seed={seed}"
        print(tag, flush=True)
        x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, fp8=True, with_do=True)
        q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
        ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
        cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
        scale = 1.0 / np.sqrt(D)
        qv, kv, vv = (oracle.e4m3_decode(b) * float(d) for b, d in zip((x.q_bits, x.k_bits, x.v_bits), x.descale))
        ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
        o = torch.from_numpy(ro).to(torch.bfloat16).cuda()
        lse = torch.from_numpy(rl).to(torch.float32).cuda()
        do = lca.bf16_from_bits(x.do_bits, "cuda")
        dq, dk, dv = lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_bwd(qv, kv, vv, x.values("do"), causal=causal, scale=scale,
                                          cu_seqlens=x.cu_seqlens, workers=None)
        errs = [rel_l2(host(g), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
        print(f"{tag}: dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
        assert max(errs) <= 5e-3, tag
