"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The kernels run on the whole seeded inputs of each workload (mid, gqa32k,
packed32k, fp8_64k). The fp64 oracle checks a seeded sample of outputs that it
can compute one by one: forward rows (O and LSE), dQ rows, and dK/dV rows of
one kv group (the oracle runs that group's full forward for the LSE and Delta
of every query row). Gradient sums that hold over whole tensors are checked
on the full GPU outputs: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per kv
head and segment (summed over the group's query heads).

Tolerances as in the small-shape tests, applied to the sampled sets: O
|err| <= max(1e-2, ulp / 2) and rel-L2 <= 5e-3, LSE <= 1e-3, gradients rel-L2
<= 1e-2 per tensor, fp8 O rel-L2 <= 5e-2.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import (TOL_FP8_REL, TOL_GRAD_REL, TOL_LSE, check_fwd, delta_from_o_rows, dev_i32, dev_u8,
                               host, max_abs, rel_l2)

pytestmark = pytest.mark.gpu


def _sample_rows(w, cu, seed, count):
    """Query/key rows: S-1, each segment's first 33 rows and last row, plus seeded uniform rows.

    A row near its segment start sees few keys, so its output is an average of few V rows: the largest
    |O| and the largest share of the bf16 rounding of P occur there."""
    must = [w.seqlen - 1]
    starts = [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])] if cu is not None else [(0, w.seqlen)]
    for a, b in starts:
        must += list(range(a, min(a + 33, b))) + [b - 1]
    return si.sample_indices(seed, w.seqlen, count, must=must)


def _sample_heads(n, seed):
    return si.sample_indices(seed + 7, n, 2, must=[0, n - 1])


def _upload(x):
    import long_context_exact_fwd_amd as lca
    return [lca.bf16_from_bits(bits, "cuda") for bits in (x.q_bits, x.k_bits, x.v_bits)]


def _forward_rows_check(w, x, o, lse, picks, tag):
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd_rows(qv, kv, vv, picks, causal=w.causal, scale=w.scale, cu_seqlens=x.cu_seqlens)
    go = np.stack([o[b, i, h] for b, h, i in picks])
    gl = np.array([lse[b, h, i] for b, h, i in picks])
    check_fwd(go, gl, ro, rl, tag=tag)
    return qv, kv, vv


def _run_fwd_bwd(name, backward):
    import torch
    import long_context_exact_fwd_amd as lca
    w = si.WORKLOADS[name]
    print(f"full-size case {name}: B={w.batch} Hq={w.hq} Hkv={w.hkv} S={w.seqlen} D={w.head_dim} causal={w.causal} "
          f"packed={w.packed} seed={w.seed} backward={backward}", flush=True)
    x = si.workload_inputs(w, with_do=backward)
    q, k, v = _upload(x)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    kw = dict(causal=w.causal, cu_seqlens=cu, scale=w.scale)
    o, lse = lca.fwd(q, k, v, **kw)
    if backward:
        do = lca.bf16_from_bits(x.do_bits, "cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(lca.bwd_workspace_bytes(w.batch, w.hq, w.hkv, w.seqlen, w.head_dim) // 4,
                         dtype=torch.float32, device="cuda")
        for ph in (lca.BWD_DELTA, lca.BWD_DKDV, lca.BWD_DQ):  # as bench.py launches them
            lca.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, phases=ph, **kw)
    torch.cuda.synchronize()
    print(f"{name}: GPU done", flush=True)
    o_h, lse_h = host(o), host(lse)
    rows = _sample_rows(w, x.cu_seqlens, w.seed, 128)
    heads = _sample_heads(w.hq, w.seed)
    picks = [(b, int(h), int(i)) for b in range(w.batch) for h in heads for i in rows]
    qv, kv, vv = _forward_rows_check(w, x, o_h, lse_h, picks, tag=f"{name} fwd ({len(picks)} rows)")
    if not backward:
        return
    dov = x.values("do")
    dq_h, dk_h, dv_h = host(dq), host(dk), host(dv)
    rq = oracle.attention_dq_rows(qv, kv, vv, dov, picks, causal=w.causal, scale=w.scale, cu_seqlens=x.cu_seqlens)
    gq = np.stack([dq_h[b, i, h] for b, h, i in picks])
    e_q = rel_l2(gq, rq)
    kvh = int(si.sample_indices(w.seed + 11, w.hkv, 1)[0])
    keys = _sample_rows(w, x.cu_seqlens, w.seed + 13, 128)
    kpicks = [(0, kvh, int(j)) for j in keys]
    rk, rv = oracle.attention_dkdv_rows(qv, kv, vv, dov, kpicks, causal=w.causal, scale=w.scale,
                                        cu_seqlens=x.cu_seqlens)
    gk = np.stack([dk_h[b, j, h] for b, h, j in kpicks])
    gv = np.stack([dv_h[b, j, h] for b, h, j in kpicks])
    e_k, e_v = rel_l2(gk, rk), rel_l2(gv, rv)
    print(f"{name} bwd sampled: dQ relL2={e_q:.3e} ({len(picks)} rows) dK relL2={e_k:.3e} dV relL2={e_v:.3e} "
          f"({len(kpicks)} keys of kv head {kvh})", flush=True)
    assert np.all(np.isfinite(dq_h)) and np.all(np.isfinite(dk_h)) and np.all(np.isfinite(dv_h))
    assert max(e_q, e_k, e_v) <= TOL_GRAD_REL
    # whole-tensor identities per kv head and segment
    G = w.hq // w.hkv
    bounds = list(zip(x.cu_seqlens[:-1], x.cu_seqlens[1:])) if x.cu_seqlens is not None else [(0, w.seqlen)]
    worst_k = worst_v = 0.0
    for b in range(w.batch):
        for h in range(w.hkv):
            for a, e in bounds:
                sk = dk_h[b, a:e, h].sum(axis=0)
                worst_k = max(worst_k, float(np.linalg.norm(sk) / np.linalg.norm(dk_h[b, a:e, h])))
                sv = dv_h[b, a:e, h].sum(axis=0)
                ref = dov[b, a:e, h * G:(h + 1) * G].sum(axis=(0, 1))
                worst_v = max(worst_v, rel_l2(sv, ref))
    print(f"{name} sums: |sum dK| / |dK| <= {worst_k:.3e}, sum dV vs sum dO relL2 <= {worst_v:.3e}", flush=True)
    # sum_j dK_j = 0 exactly; bf16 rounding of each row leaves noise far below the norm of dK itself
    assert worst_k <= 1e-2 and worst_v <= 1e-2


def test_mid_full_forward_sampled():
    """B=2, H=32, S=8192, D=128 causal forward."""
    _run_fwd_bwd("mid", backward=False)


def test_gqa32k_full_forward_backward_sampled():
    """B=1, Hq=28, Hkv=4, S=32768, D=128 causal forward + backward (the bench workload)."""
    _run_fwd_bwd("gqa32k", backward=True)


def test_packed32k_full_forward_backward_sampled():
    """B=1, Hq=14, Hkv=2, S=32768 packed (seed-4 lengths), D=128 causal forward + backward."""
    _run_fwd_bwd("packed32k", backward=True)


def test_fp8_64k_full_forward_sampled():
    """B=1, Hq=8, Hkv=1, S=65536, D=128 causal fp8 forward, O bf16 and LSE fp32."""
    import torch
    import long_context_exact_fwd_amd as lca
    w = si.WORKLOADS["fp8_64k"]
    print(f"full-size case fp8_64k: Hq={w.hq} Hkv={w.hkv} S={w.seqlen} seed={w.seed}", flush=True)
    x = si.workload_inputs(w)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o_h, lse_h = host(o), host(lse)
    rows = _sample_rows(w, None, w.seed, 128)
    heads = _sample_heads(w.hq, w.seed)
    picks = [(0, int(h), int(i)) for h in heads for i in rows]
    qv = oracle.e4m3_decode(x.q_bits) * float(x.descale[0])
    kv = oracle.e4m3_decode(x.k_bits) * float(x.descale[1])
    vv = oracle.e4m3_decode(x.v_bits) * float(x.descale[2])
    ro, rl = oracle.attention_fwd_rows(qv, kv, vv, picks, causal=True, scale=w.scale)
    go = np.stack([o_h[0, i, h] for _, h, i in picks])
    gl = np.array([lse_h[0, h, i] for _, h, i in picks])
    rr, rlse = rel_l2(go, ro), max_abs(gl, rl)
    print(f"fp8_64k sampled ({len(picks)} rows): O relL2={rr:.3e} LSE maxabs={rlse:.3e}", flush=True)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h))
    assert rr <= TOL_FP8_REL and rlse <= TOL_LSE


def test_long_sequence_256k_sampled():
    """B=1, Hq=2, Hkv=1, S=262144, D=128 causal fwd + bwd: the longest sequence tested, for the 32-bit
    row and byte arithmetic of the kernels. Forward and dQ on sampled rows; dK/dV through the whole-tensor
    identities (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i), which involve every key row."""
    import torch
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D, seed = 1, 2, 1, 262144, 128, 21
    print(f"long case: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal seed={seed}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed)
    q, k, v = _upload(x)
    do = lca.bf16_from_bits(x.do_bits, "cuda")
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    print("long case: GPU done", flush=True)
    o_h, lse_h, dq_h, dk_h, dv_h = host(o), host(lse), host(dq), host(dk), host(dv)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(dq_h)) and np.all(np.isfinite(dk_h))
    rows = si.sample_indices(seed, S, 48, must=[0, 1, 65535, 65536, 131071, 131072, S - 2, S - 1])
    picks = [(0, h, int(i)) for h in range(Hq) for i in rows]
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd_rows(qv, kv, vv, picks, causal=True, scale=scale)
    check_fwd(np.stack([o_h[0, i, h] for _, h, i in picks]), np.array([lse_h[0, h, i] for _, h, i in picks]),
              ro, rl, tag=f"long fwd ({len(picks)} rows)")
    dov = x.values("do")
    rq = oracle.attention_dq_rows(qv, kv, vv, dov, picks, causal=True, scale=scale)
    gq = np.stack([dq_h[0, i, h] for _, h, i in picks])
    e_q = rel_l2(gq, rq)
    # the same rows against the oracle's dQ given the kernel's bf16 O (Delta = dO . O with that O enters
    # dS linearly: dQ_i moves by -scale eps_i sum_j P_ij K_j, eps_i = dO_i . (O_given - O)_i, in the rows
    # that see at least 64 keys; the first 63 take Delta from its definition)
    kbar, _ = oracle.attention_fwd_rows(qv, kv, kv, picks, causal=True, scale=scale)
    go = np.stack([o_h[0, i, h] for _, h, i in picks])
    eps = np.einsum("nd,nd->n", np.stack([dov[0, i, h] for _, h, i in picks]), go - ro)[:, None]
    eps *= delta_from_o_rows(S, True)[[i for _, _, i in picks]][:, None]
    e_q_given = rel_l2(gq, rq - scale * eps * kbar)
    sk = dk_h[0, :, 0].sum(axis=0)
    e_k = float(np.linalg.norm(sk) / np.linalg.norm(dk_h[0, :, 0]))
    e_v = rel_l2(dv_h[0, :, 0].sum(axis=0), dov[0, :, :].sum(axis=(0, 1)))
    print(f"long bwd: dQ relL2={e_q:.3e} ({len(picks)} rows; {e_q_given:.3e} against the dQ given the kernel's "
          f"O); |sum dK|/|dK|={e_k:.3e}; sum dV vs sum dO relL2={e_v:.3e}", flush=True)
    assert e_q <= TOL_GRAD_REL and e_q_given <= TOL_GRAD_REL and e_k <= 1e-2 and e_v <= 1e-2


def test_fp8_64k_full_forward_backward_sampled():
    """B=1, Hq=8, Hkv=1, S=65536, D=128 causal fp8 forward then its backward (attn_bwd_fp8), as bench.py's
    fp8_64k_fwd_bwd workload runs them. dQ on sampled rows against the oracle on the dequantised inputs, at
    the fp8 bound (the forward's fp8 probabilities reach the gradient through Delta = dO . O); whole-tensor
    sums: sum_j dV_j = sum_i dO_i (exact for any O) and |sum_j dK_j| small against |dK|."""
    import torch
    import long_context_exact_fwd_amd as lca
    w = si.WORKLOADS["fp8_64k"]
    print(f"full-size case fp8_64k fwd+bwd: Hq={w.hq} Hkv={w.hkv} S={w.seqlen} seed={w.seed}", flush=True)
    x = si.workload_inputs(w, with_do=True)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    do = lca.bf16_from_bits(x.do_bits, "cuda")
    o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=True, scale=w.scale)
    dq, dk, dv = lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    print("fp8_64k fwd+bwd: GPU done", flush=True)
    dq_h, dk_h, dv_h = host(dq), host(dk), host(dv)
    assert np.all(np.isfinite(dq_h)) and np.all(np.isfinite(dk_h)) and np.all(np.isfinite(dv_h))
    rows = _sample_rows(w, None, w.seed, 64)
    picks = [(0, h, int(i)) for h in _sample_heads(w.hq, w.seed) for i in rows]
    qv = oracle.e4m3_decode(x.q_bits) * float(x.descale[0])
    kv = oracle.e4m3_decode(x.k_bits) * float(x.descale[1])
    vv = oracle.e4m3_decode(x.v_bits) * float(x.descale[2])
    dov = x.values("do")
    rq = oracle.attention_dq_rows(qv, kv, vv, dov, picks, causal=True, scale=w.scale)
    e_q = rel_l2(np.stack([dq_h[0, i, h] for _, h, i in picks]), rq)
    sk = float(np.linalg.norm(dk_h[0, :, 0].sum(axis=0)) / np.linalg.norm(dk_h[0, :, 0]))
    sv = rel_l2(dv_h[0, :, 0].sum(axis=0), dov[0].sum(axis=(0, 1)))
    print(f"fp8_64k bwd: dQ relL2={e_q:.3e} ({len(picks)} rows); |sum dK|/|dK|={sk:.3e}; sum dV vs sum dO "
          f"relL2={sv:.3e}", flush=True)
    assert e_q <= TOL_FP8_REL and sk <= TOL_FP8_REL and sv <= 1e-2


def test_ring4_gqa32k_full_forward_backward_sampled():
    """The gqa32k workload as a 4-chunk Ring-Attention pass on one GPU, as bench.py times it: the forward with
    attn_fwd_merge per (query chunk, key chunk <= it) and the backward with attn_bwd_accumulate per pair.
    Sampled forward rows, dQ rows and one kv group's dK/dV keys against the oracle (bars as above), and the
    whole fp32 gradients against the one-shot attn_bwd (rel-L2 <= 1e-2 per tensor)."""
    import torch
    import long_context_exact_fwd_amd as lca
    from tests.test_parity_ring import ring_backward_accumulate, ring_forward_fused
    w = si.WORKLOADS["gqa32k"]
    nchunk = 4
    print(f"full-size ring case gqa32k in {nchunk} chunks: B={w.batch} Hq={w.hq} Hkv={w.hkv} S={w.seqlen}", flush=True)
    x = si.workload_inputs(w, with_do=True)
    q, k, v = _upload(x)
    do = lca.bf16_from_bits(x.do_bits, "cuda")
    o, lse = ring_forward_fused(q, k, v, nchunk, True, w.scale)
    dq, dk, dv = ring_backward_accumulate(q, k, v, o, lse, do, nchunk, True, w.scale)
    gq1, gk1, gv1 = lca.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    print("ring gqa32k: GPU done", flush=True)
    o_h, lse_h = host(o), host(lse)
    rows = _sample_rows(w, None, w.seed + 21, 128)
    # rows around each chunk boundary too: their first key chunk is the diagonal one
    L = w.seqlen // nchunk
    rows = np.unique(np.concatenate([rows, [r * L + d for r in range(1, nchunk) for d in (-1, 0, 1, 63, 64)]]))
    heads = _sample_heads(w.hq, w.seed + 21)
    picks = [(0, int(h), int(i)) for h in heads for i in rows]
    qv, kv, vv = _forward_rows_check(w, x, o_h, lse_h, picks, tag=f"ring gqa32k fwd ({len(picks)} rows)")
    dov = x.values("do")
    dq_h, dk_h, dv_h = host(dq), host(dk), host(dv)
    rq = oracle.attention_dq_rows(qv, kv, vv, dov, picks, causal=True, scale=w.scale)
    e_q = rel_l2(np.stack([dq_h[b, i, h] for b, h, i in picks]), rq)
    kvh = int(si.sample_indices(w.seed + 23, w.hkv, 1)[0])
    keys = _sample_rows(w, None, w.seed + 25, 128)
    kpicks = [(0, kvh, int(j)) for j in keys]
    rk, rv = oracle.attention_dkdv_rows(qv, kv, vv, dov, kpicks, causal=True, scale=w.scale)
    e_k = rel_l2(np.stack([dk_h[b, j, h] for b, h, j in kpicks]), rk)
    e_v = rel_l2(np.stack([dv_h[b, j, h] for b, h, j in kpicks]), rv)
    one = [rel_l2(a, host(r)) for a, r in ((dq_h, gq1), (dk_h, gk1), (dv_h, gv1))]
    print(f"ring gqa32k bwd sampled: dQ relL2={e_q:.3e} dK relL2={e_k:.3e} dV relL2={e_v:.3e}; against the one-shot "
          f"backward: dQ {one[0]:.3e} dK {one[1]:.3e} dV {one[2]:.3e}", flush=True)
    assert np.all(np.isfinite(dq_h)) and np.all(np.isfinite(dk_h)) and np.all(np.isfinite(dv_h))
    assert max(e_q, e_k, e_v) <= TOL_GRAD_REL and max(one) <= TOL_GRAD_REL
