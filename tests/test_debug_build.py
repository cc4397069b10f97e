"""GPU: the debug library (libmi355attn_debug.so, the sources compiled with
-DATTN_DEBUG) runs every entry point with its LDS accesses bounds-checked on
the device. Each case runs once through the release library and once through
the debug one: the debug call must return ATTN_OK (no access failed its check;
a failure would raise ATTN_ERR_DEBUG_CHECK) and give bitwise the release
outputs, since the checks change no arithmetic. The cases cover both block
geometries of the forward and of the dQ pass, key and head splits, packed
segments with few-key rows, the ring-merge forwards, fp8, the fp32
accumulating backward and the no-allocation backward.
"""
import os

import numpy as np
import pytest

import seeded_inputs as si
from tests.gpu_helpers import dev_bf16, dev_i32, dev_u8

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not os.path.exists(os.path.join(os.path.dirname(os.path.dirname(
                  os.path.abspath(__file__))), "long_context_exact_fwd_amd", "libmi355attn_debug.so")),
                  reason="debug library not built")]


def _both(fn):
    """fn() through the release library, then through the debug library; outputs bitwise equal."""
    import torch
    import long_context_exact_fwd_amd as lca
    try:
        lca.use_debug_library(False)
        ref = [t.clone() for t in fn()]
        torch.cuda.synchronize()
        lca.use_debug_library(True)
        got = [t.clone() for t in fn()]
        torch.cuda.synchronize()
    finally:
        lca.use_debug_library(False)
    assert len(ref) == len(got)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), f"output {i} differs between the release and the debug library"


def _bf16(B, Hq, Hkv, S, D, lengths, seed=61):
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, with_do=True)
    q, k, v, do = (dev_bf16(b) for b in (x.q_bits, x.k_bits, x.v_bits, x.do_bits))
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    return q, k, v, do, cu


FWD = [
    # B, Hq, Hkv, S, D, causal, lengths
    (1, 4, 2, 1000, 128, True, None),
    (2, 3, 1, 700, 64, False, None),
    (1, 7, 1, 1000, 128, True, [100, 1, 1, 64, 65, 500, 269]),
    (1, 2, 1, 4500, 64, False, [4000, 500]),
    (1, 1, 1, 8192, 128, True, None),  # key split
]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", FWD)
def test_forward_and_merge_under_the_debug_build(B, Hq, Hkv, S, D, causal, lengths, waves, monkeypatch):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"debug fwd B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} waves={waves}",
          flush=True)
    monkeypatch.setenv("ATTN_FWD_WAVES", waves)
    q, k, v, _, cu = _bf16(B, Hq, Hkv, S, D, lengths)
    _both(lambda: lca.fwd(q, k, v, causal=causal, cu_seqlens=cu))

    def ring_step():
        o_acc = torch.zeros((B, S, Hq, D), dtype=torch.float32, device="cuda")
        l_acc = torch.zeros((B, Hq, S), dtype=torch.float32, device="cuda")
        o_out = torch.empty_like(q)
        lca.fwd_merge(q, k, v, o_acc, l_acc, causal=causal, accumulate=False, cu_seqlens=cu)
        lca.fwd_merge(q, k, v, o_acc, l_acc, causal=False, accumulate=True, o_out=o_out, cu_seqlens=cu)
        return o_acc, l_acc, o_out
    _both(ring_step)


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [(1, 4, 2, 1000, True, None),
                                                       (1, 2, 2, 700, False, [1, 299, 400]),
                                                       (1, 1, 1, 8192, True, None)])
def test_fp8_forward_and_merge_under_the_debug_build(B, Hq, Hkv, S, causal, lengths, waves, monkeypatch):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"debug fp8 fwd B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths} waves={waves}", flush=True)
    monkeypatch.setenv("ATTN_FWD_WAVES", waves)
    D = 128
    x = si.make_inputs(B, Hq, Hkv, S, D, 67, lengths=lengths, fp8=True, with_do=False)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    _both(lambda: lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu))

    def ring_step():
        o_acc = torch.zeros((B, S, Hq, D), dtype=torch.float32, device="cuda")
        l_acc = torch.zeros((B, Hq, S), dtype=torch.float32, device="cuda")
        lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, l_acc, causal=causal, accumulate=False, cu_seqlens=cu)
        lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, l_acc, causal=False, accumulate=True, cu_seqlens=cu)
        return o_acc, l_acc
    _both(ring_step)


def test_merge_under_the_debug_build():
    import torch
    import long_context_exact_fwd_amd as lca
    print("debug merge", flush=True)
    q, k, v, _, _ = _bf16(1, 4, 2, 1000, 128, None)
    o, lse = lca.fwd(q, k, v, causal=True)

    def run():
        o_acc = torch.zeros(o.shape, dtype=torch.float32, device="cuda")
        l_acc = torch.zeros(lse.shape, dtype=torch.float32, device="cuda")
        out = torch.empty_like(o)
        lca.merge(o_acc, l_acc, o, lse, accumulate=False)
        lca.merge(o_acc, l_acc, o, lse, accumulate=True, o_out=out)
        return o_acc, l_acc, out
    _both(run)


BWD = [
    # B, Hq, Hkv, S, D, causal, lengths
    (1, 4, 2, 1000, 128, True, None),  # head and key splits
    (2, 3, 1, 700, 64, False, None),
    (1, 7, 1, 1000, 128, True, [100, 1, 1, 64, 65, 500, 269]),
    (4, 32, 2, 1000, 128, True, None),  # no split: the dQ geometry override applies
]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", BWD)
def test_backward_under_the_debug_build(B, Hq, Hkv, S, D, causal, lengths, waves, monkeypatch):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"debug bwd B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} dq waves={waves}",
          flush=True)
    monkeypatch.setenv("ATTN_DQ_WAVES", waves)
    q, k, v, do, cu = _bf16(B, Hq, Hkv, S, D, lengths)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu)
    torch.cuda.synchronize()
    _both(lambda: lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu))

    def accumulate():
        acc = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (q, k, v)]
        lca.bwd_accumulate(q, k, v, o, lse, do, *acc, causal=causal, accumulate=False, cu_seqlens=cu)
        lca.bwd_accumulate(q, k, v, o, lse, do, *acc, causal=causal, accumulate=True, cu_seqlens=cu)
        return acc
    _both(accumulate)
    _both(lambda: lca.bwd_noalloc(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu))


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths", [(1, 4, 2, 1000, True, None),
                                                       (1, 2, 2, 700, False, [1, 299, 400])])
def test_fp8_backward_under_the_debug_build(B, Hq, Hkv, S, causal, lengths):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"debug fp8 bwd B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths}", flush=True)
    D = 128
    x = si.make_inputs(B, Hq, Hkv, S, D, 71, lengths=lengths, fp8=True, with_do=True)
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    do = dev_bf16(x.do_bits)
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd_fp8(q8, k8, v8, *ds, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    _both(lambda: lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale))
