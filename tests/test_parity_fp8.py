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
