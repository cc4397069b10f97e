"""GPU parity of both dQ block geometries: 128-query blocks of 4 waves and
256-query blocks of 8 waves that share each K/V tile (ATTN_DQ_WAVES=4|8).

The shapes give at least 1024 dQ workgroups of 128 queries, so the key tiles
are not split (a split dQ always runs 4 waves) and the override takes effect.
Each geometry meets the oracle bar (rel-L2 <= 1e-2 per gradient), and the two
agree bitwise: every query row visits its key tiles in the same order, and the
tiles the taller block adds for some rows are fully masked for them, adding
exact zeros. The bf16, fp32-accumulating and fp8 entry points are covered.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import check_grads, dev_bf16, dev_i32, dev_u8, host

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, S, D, causal, lengths: B * Hq * ceil(S / 128) >= 1024
    (4, 32, 2, 1000, 128, True, None),
    (4, 32, 2, 1000, 128, False, None),
    (1, 64, 8, 2048, 128, True, [100, 1, 1, 64, 65, 500, 1317]),
    (8, 16, 2, 1000, 64, False, None),
]


def _inputs(B, Hq, Hkv, S, D, causal, lengths):
    import torch
    import long_context_exact_fwd_amd as lca
    x = si.make_inputs(B, Hq, Hkv, S, D, 53, lengths=lengths, with_do=True)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    return x, (q, k, v, o, lse, do), cu, scale


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", CASES)
def test_dq_block_geometries_match_oracle_and_each_other(B, Hq, Hkv, S, D, causal, lengths, monkeypatch):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"dq geometry case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
    x, args, cu, scale = _inputs(B, Hq, Hkv, S, D, causal, lengths)
    rq, rk, rv = oracle.attention_bwd(x.values("q"), x.values("k"), x.values("v"), x.values("do"), causal=causal,
                                      scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    outs, accs = [], []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_DQ_WAVES", waves)
        dq, dk, dv = lca.bwd(*args, causal=causal, cu_seqlens=cu, scale=scale)
        torch.cuda.synchronize()
        check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)], tag=f"bwd dq waves={waves}")
        outs.append((dq, dk, dv))
        # fp32 accumulators: written by a first call, added to by a second
        q, k, v = args[:3]
        acc = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (q, k, v)]
        lca.bwd_accumulate(*args, *acc, causal=causal, accumulate=False, cu_seqlens=cu, scale=scale)
        lca.bwd_accumulate(*args, *acc, causal=causal, accumulate=True, cu_seqlens=cu, scale=scale)
        torch.cuda.synchronize()
        accs.append(acc)
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(accs[0], accs[1]):
        assert torch.equal(a, b)
    # twice the one-call gradient, to fp32 rounding of the sum
    check_grads([("dQ acc", host(accs[1][0]) / 2, rq)], tag="bwd_accumulate dq waves=8")


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [(4, 32, 2, 1000, True, None),
                                                       (1, 64, 8, 2048, False, [700, 1, 1347])])
def test_fp8_backward_dq_block_geometries(B, Hq, Hkv, S, causal, lengths, monkeypatch):
    """attn_bwd_fp8 with both dQ geometries, given the exact O and LSE: the oracle's gradient bar and bitwise
    agreement."""
    import torch
    import long_context_exact_fwd_amd as lca
    D = 128
    print(f"fp8 dq geometry case B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 59, lengths=lengths, fp8=True, with_do=True)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    do = dev_bf16(x.do_bits)
    scale = 1.0 / np.sqrt(D)
    qv = oracle.e4m3_decode(x.q_bits) * float(x.descale[0])
    kv = oracle.e4m3_decode(x.k_bits) * float(x.descale[1])
    vv = oracle.e4m3_decode(x.v_bits) * float(x.descale[2])
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    o = torch.from_numpy(ro).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(rl).to(torch.float32).cuda()
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, x.values("do"), causal=causal, scale=scale,
                                      cu_seqlens=x.cu_seqlens, workers=None)
    outs = []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_DQ_WAVES", waves)
        dq, dk, dv = lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
        torch.cuda.synchronize()
        check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)],
                    tag=f"fp8 bwd dq waves={waves}")
        outs.append((dq, dk, dv))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
