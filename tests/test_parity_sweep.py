"""A seeded sweep of small random shapes through every bf16 entry point, against the fp64 oracle.

Each case draws batch, GQA group, kv heads, sequence length (ragged, from 1),
head dim, mask and (for batch 1) a random packing, then checks through the
C ABI:
* attn_fwd: O and LSE to the forward bar (check_fwd);
* attn_bwd: dQ, dK, dV rel-L2 <= 1e-2 (check_grads);
* attn_fwd_merge: one ring step into a random running result, against the
  oracle's merge;
* attn_bwd_accumulate (accumulate off): rounds to attn_bwd's output bit for bit;
and the head-dim-128 draws through attn_fwd_fp8, attn_bwd_fp8 and
attn_fwd_fp8_merge against the oracle on the dequantised inputs.
The draws are fixed by the seed, so a failure names a reproducible case.
ATTN_SWEEP_CASES=N widens the sweep to the first N draws.
"""
import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import check_fwd, check_grads, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 3, 4, 7]))
    S = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 300)), int(rng.integers(300, 700))]))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    lengths = None
    B = int(rng.integers(1, 3))
    if S >= 8 and rng.integers(0, 2) == 1:
        B = 1
        n = int(rng.integers(2, min(6, S) + 1))
        cuts = np.sort(rng.choice(np.arange(1, S), size=n - 1, replace=False))
        edges = np.concatenate([[0], cuts, [S]])
        lengths = [int(b - a) for a, b in zip(edges[:-1], edges[1:])]
    return B, g * hkv, hkv, S, D, causal, lengths


# 24 cases by default; ATTN_SWEEP_CASES=N runs the first N draws (the same 24 first)
CASES = [_draw(i) for i in range(int(os.environ.get("ATTN_SWEEP_CASES", "24")))]


# draws past the default 24 that failed a wider sweep once, kept as regression cases
REGRESSION = [
    457,  # S=2 causal, D=64: Delta from the bf16 O dominated dP - Delta (fixed by Delta from its definition)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sweep_case(case):
    _sweep_case(case, CASES[case])


@pytest.mark.parametrize("draw", REGRESSION)
def test_sweep_regression(draw):
    _sweep_case(draw, _draw(draw))


def _sweep_case(case, shape):
    import torch
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D, causal, lengths = shape
    print(f"sweep {case}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=2000 + case, lengths=lengths)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    check_fwd(host(o), host(lse), ro, rl, tag="fwd")
    grads = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, dov, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens,
                                      workers=None)
    check_grads([("dQ", host(grads[0]), rq), ("dK", host(grads[1]), rk), ("dV", host(grads[2]), rv)], tag="bwd")
    acc = [torch.empty(t.shape, dtype=torch.float32, device=t.device) for t in grads]
    lca.bwd_accumulate(q, k, v, o, lse, do, *acc, causal=causal, accumulate=False, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    for a, r in zip(acc, grads):
        assert torch.equal(a.to(torch.bfloat16), r)
    rng = np.random.default_rng(3000 + case)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l1 = rng.uniform(-2.0, 8.0, (B, Hq, S)).astype(np.float32)
    o_acc = torch.from_numpy(o1.copy()).cuda()
    l_acc = torch.from_numpy(l1.copy()).cuda()
    lca.fwd_merge(q, k, v, o_acc, l_acc, causal=causal, accumulate=True, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_partials(o1.astype(np.float64), l1.astype(np.float64), ro, rl)
    check_fwd(host(o_acc), host(l_acc), mo, ml, tag="fwd_merge")


FP8_CASES = [c for c in CASES if c[4] == 128][: max(8, len(CASES) // 3)]


def _fp8_draw(j):
    """The j-th head-dim-128 draw: FP8_CASES[j] of a sweep wide enough to hold it."""
    i = -1
    while j >= 0:
        i += 1
        if _draw(i)[4] == 128:
            j -= 1
    return _draw(i)


FP8_REGRESSION = [
    319,  # S=2 causal: as draw 457 of the bf16 sweep
]


@pytest.mark.parametrize("case", range(len(FP8_CASES)))
def test_sweep_fp8_case(case):
    """The head-dim-128 draws through the fp8 entry points: attn_fwd_fp8 (O rel-L2 <= 5e-2, LSE <= 1e-3),
    attn_bwd_fp8 from the exact O (rel-L2 <= 1e-2) and attn_fwd_fp8_merge (fp8 bounds), against the oracle on the
    dequantised inputs."""
    _sweep_fp8_case(case, FP8_CASES[case])


@pytest.mark.parametrize("case", FP8_REGRESSION)
def test_sweep_fp8_regression(case):
    _sweep_fp8_case(case, _fp8_draw(case))


def _sweep_fp8_case(case, shape):
    import torch
    import long_context_exact_fwd_amd as lca
    from tests.gpu_helpers import TOL_FP8_REL, TOL_LSE, TOL_ZERO_GRAD_ABS, dev_u8, max_abs, rel_l2
    B, Hq, Hkv, S, D, causal, lengths = shape
    print(f"fp8 sweep {case}: B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=4000 + case, lengths=lengths, fp8=True)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    qv, kv, vv = (oracle.e4m3_decode(b) * float(d) for b, d in zip((x.q_bits, x.k_bits, x.v_bits), x.descale))
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    e_o, e_l = rel_l2(host(o), ro), max_abs(host(lse), rl)
    print(f"fp8 fwd O relL2={e_o:.3e} LSE maxabs={e_l:.3e}", flush=True)
    assert e_o <= TOL_FP8_REL and e_l <= TOL_LSE
    # backward from the exact O rounded to bf16 and the exact LSE: the gradient of the dequantised attention
    o_ex = torch.from_numpy(ro).to(torch.bfloat16).cuda()
    lse_ex = torch.from_numpy(rl).to(torch.float32).cuda()
    do = dev_bf16(x.do_bits)
    dq, dk, dv = lca.bwd_fp8(q8, k8, v8, *ds, o_ex, lse_ex, do, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    dov = x.values("do")
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, dov, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens,
                                      workers=None)
    if np.any(rq != 0):
        check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)], tag="fp8 bwd")
    else:
        # every row sees one key (S = 1 or segments of length 1 with the causal mask): the exact dQ and dK are
        # zero. These rows take Delta = P dP from its definition (not dO . O from the bf16 O, whose rounding of
        # the dequantised values would otherwise show), with P = 1 up to fp32 rounding, so dS is fp32 noise
        # and dQ, dK stay within the zero-reference bound of 1e-3.
        e_q, e_k, e_v = max_abs(host(dq), rq), max_abs(host(dk), rk), rel_l2(host(dv), rv)
        print(f"fp8 bwd (one key per row): dQ maxabs={e_q:.3e} dK maxabs={e_k:.3e}, dV relL2={e_v:.3e}", flush=True)
        assert e_q <= TOL_ZERO_GRAD_ABS and e_k <= TOL_ZERO_GRAD_ABS and e_v <= 1e-2
    rng = np.random.default_rng(5000 + case)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l1 = rng.uniform(-2.0, 8.0, (B, Hq, S)).astype(np.float32)
    o_acc, l_acc = torch.from_numpy(o1.copy()).cuda(), torch.from_numpy(l1.copy()).cuda()
    lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, l_acc, causal=causal, accumulate=True, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_partials(o1.astype(np.float64), l1.astype(np.float64), ro, rl)
    e_mo, e_ml = rel_l2(host(o_acc), mo), max_abs(host(l_acc), ml)
    print(f"fp8 fwd_merge O relL2={e_mo:.3e} LSE maxabs={e_ml:.3e}", flush=True)
    assert e_mo <= TOL_FP8_REL and e_ml <= TOL_LSE


# Stress draws: the same random shapes with Q and K scaled (peaky softmax rows: the forward's running maximum
# moves past the first tile's, the backward's rows are dominated by a few keys). Outside the stated workloads,
# so O is held to the bound of the kernel's rounding (rounding_o_bound) and the fp8 LSE to fp8_lse_bound; the
# gradients keep the general 1e-2 (the worst of 1200 such draws: dQ 9.1e-3, dK 9.2e-3; fp8 backward from the
# exact O, 299 draws: 8.0e-3).
# ATTN_STRESS_CASES=N runs the first N.
STRESS = [(_draw(10000 + i), (2.5, 3.0, 4.0)[i % 3]) for i in range(int(os.environ.get("ATTN_STRESS_CASES", "12")))]


@pytest.mark.parametrize("case", range(len(STRESS)))
def test_sweep_stress_case(case):
    import torch
    import long_context_exact_fwd_amd as lca
    from tests.gpu_helpers import TOL_FP8_REL, dev_u8, fp8_lse_bound, max_abs, rel_l2, rounding_o_bound
    (B, Hq, Hkv, S, D, causal, lengths), qk_std = STRESS[case]
    print(f"stress {case}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} qk_std={qk_std}",
          flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=20000 + case, lengths=lengths, qk_std=qk_std)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    abar, _ = oracle.attention_fwd(qv, kv, np.abs(vv), causal=causal, scale=scale, cu_seqlens=x.cu_seqlens,
                                   workers=None)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    grads = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    check_fwd(host(o), host(lse), ro, rl, tag="stress fwd", bound=rounding_o_bound(host(o), ro, abar))
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, dov, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens,
                                      workers=None)
    check_grads([("dQ", host(grads[0]), rq), ("dK", host(grads[1]), rk), ("dV", host(grads[2]), rv)],
                tag="stress bwd")
    if D != 128:
        return
    x8 = si.make_inputs(B, Hq, Hkv, S, D, seed=30000 + case, lengths=lengths, fp8=True, qk_std=qk_std,
                        with_do=True)
    q8, k8, v8 = dev_u8(x8.q_bits), dev_u8(x8.k_bits), dev_u8(x8.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x8.descale]
    qv8, kv8, vv8 = (oracle.e4m3_decode(b) * float(d) for b, d in zip((x8.q_bits, x8.k_bits, x8.v_bits), x8.descale))
    ro8, rl8 = oracle.attention_fwd(qv8, kv8, vv8, causal=causal, scale=scale, cu_seqlens=x8.cu_seqlens,
                                    workers=None)
    o8, l8 = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    e_o = rel_l2(host(o8), ro8)
    worst = float(np.max(np.abs(host(l8) - rl8) / fp8_lse_bound(qv8, kv8, causal, scale, x8.cu_seqlens)))
    print(f"stress fp8 fwd O relL2={e_o:.3e} LSE maxabs={max_abs(host(l8), rl8):.3e} ({worst:.2f} of its bound)",
          flush=True)
    assert np.all(np.isfinite(host(o8))) and e_o <= TOL_FP8_REL and worst <= 1.0
    # attn_bwd_fp8 from the exact O (bf16) and LSE: the exact gradient of the dequantised inputs (the worst of 299
    # such draws: rel-L2 8.0e-3)
    o_ex = torch.from_numpy(ro8).to(torch.bfloat16).cuda()
    lse_ex = torch.from_numpy(rl8).to(torch.float32).cuda()
    g8 = lca.bwd_fp8(q8, k8, v8, *ds, o_ex, lse_ex, dev_bf16(x8.do_bits), causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    rq8, rk8, rv8 = oracle.attention_bwd(qv8, kv8, vv8, x8.values("do"), causal=causal, scale=scale,
                                         cu_seqlens=x8.cu_seqlens, workers=None)
    check_grads([("dQ", host(g8[0]), rq8), ("dK", host(g8[1]), rk8), ("dV", host(g8[2]), rv8)], tag="stress fp8 bwd")
