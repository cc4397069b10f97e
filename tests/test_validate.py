"""ATTN_VALIDATE=1: malformed cu_seqlens arrays are rejected on the host before
anything is launched (no kernel ever sees them here), by every entry point that
takes one; a valid array gives the same bits as an unvalidated call."""
import numpy as np
import pytest

import seeded_inputs as si
from tests.gpu_helpers import dev_bf16, dev_i32, dev_u8

pytestmark = pytest.mark.gpu

BAD = [
    [0, 100, 100, 256],  # empty segment
    [1, 100, 256],       # does not start at 0
    [0, 100, 300],       # ends past seqlen
    [0, 100, 200],       # ends before seqlen
    [0, 200, 100, 256],  # decreasing
]


def test_validate_rejects_malformed_cu_seqlens(monkeypatch):
    import torch
    import long_context_exact_fwd_amd as lca
    S = 256
    x = si.make_inputs(1, 2, 1, S, 128, 31, lengths=[100, 156], with_do=True)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    good = dev_i32(x.cu_seqlens)
    o_ref, l_ref = lca.fwd(q, k, v, causal=True, cu_seqlens=good)
    g_ref = lca.bwd(q, k, v, o_ref, l_ref, do, causal=True, cu_seqlens=good)
    torch.cuda.synchronize()
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    o, lse = lca.fwd(q, k, v, causal=True, cu_seqlens=good)
    g = lca.bwd(q, k, v, o, lse, do, causal=True, cu_seqlens=good)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert all(torch.equal(a, b) for a, b in zip(g, g_ref))
    x8 = si.make_inputs(1, 2, 1, S, 128, 32, lengths=[100, 156], fp8=True, with_do=False)
    q8, k8, v8 = dev_u8(x8.q_bits), dev_u8(x8.k_bits), dev_u8(x8.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x8.descale]
    for bad in BAD:
        print(f"case malformed cu_seqlens {bad}", flush=True)
        cu = dev_i32(np.array(bad, dtype=np.int32))
        o_acc = torch.zeros((1, S, 2, 128), dtype=torch.float32, device="cuda")
        l_acc = torch.zeros((1, 2, S), dtype=torch.float32, device="cuda")
        calls = [lambda: lca.fwd(q, k, v, causal=True, cu_seqlens=cu),
                 lambda: lca.fwd_fp8(q8, k8, v8, *ds, causal=True, cu_seqlens=cu),
                 lambda: lca.fwd_merge(q, k, v, o_acc, l_acc, causal=True, cu_seqlens=cu),
                 lambda: lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, l_acc, causal=True, cu_seqlens=cu),
                 lambda: lca.bwd(q, k, v, o, lse, do, causal=True, cu_seqlens=cu),
                 lambda: lca.bwd_noalloc(q, k, v, o, lse, do, causal=True, cu_seqlens=cu),
                 lambda: lca.bwd_accumulate(q, k, v, o, lse, do, torch.zeros_like(q, dtype=torch.float32),
                                            torch.zeros_like(k, dtype=torch.float32),
                                            torch.zeros_like(v, dtype=torch.float32), causal=True, cu_seqlens=cu),
                 lambda: lca.bwd_fp8(q8, k8, v8, *ds, o, lse, do, causal=True, cu_seqlens=cu)]
        for call in calls:
            with pytest.raises(lca.AttnError) as err:
                call()
            assert err.value.status == lca.ATTN_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def test_binding_rejects_tensors_that_do_not_fit_the_sizes():
    """The C ABI takes bare pointers, so the binding checks every tensor against the call's sizes before the
    call: a smaller or differently typed tensor would otherwise be read or written past its end."""
    import torch
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D = 1, 4, 2, 128, 64
    x = si.make_inputs(B, Hq, Hkv, S, D, 33, with_do=True)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    o, lse = lca.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    short_v = v[:, : S // 2].contiguous()
    bad_o = torch.empty((B, S, Hq, D // 2), dtype=torch.bfloat16, device="cuda")
    bad_lse = torch.empty((B, Hq, S // 2), dtype=torch.float32, device="cuda")
    f32 = lambda t: torch.zeros(t.shape, dtype=torch.float32, device="cuda")  # noqa: E731
    x8 = si.make_inputs(B, Hq, Hkv, S, 128, 34, fp8=True, with_do=False)
    q8, k8, v8 = dev_u8(x8.q_bits), dev_u8(x8.k_bits), dev_u8(x8.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x8.descale]
    empty = torch.empty(0, dtype=torch.float32, device="cuda")
    calls = {
        "v shorter than k": lambda: lca.fwd(q, k, short_v, causal=True),
        "fwd out of the wrong shape": lambda: lca.fwd(q, k, v, causal=True, out=bad_o),
        "fwd lse of the wrong shape": lambda: lca.fwd(q, k, v, causal=True, lse=bad_lse),
        "fwd out of the wrong dtype": lambda: lca.fwd(q, k, v, causal=True, out=f32(o)),
        "bwd o of the wrong shape": lambda: lca.bwd(q, k, v, bad_o, lse, do, causal=True),
        "bwd lse of the wrong shape": lambda: lca.bwd(q, k, v, o, bad_lse, do, causal=True),
        "bwd dq of the wrong shape": lambda: lca.bwd(q, k, v, o, lse, do, causal=True, dq=bad_o),
        "bwd_noalloc do of the wrong shape": lambda: lca.bwd_noalloc(q, k, v, o, lse, bad_o, causal=True),
        "bwd_accumulate dk_acc of the wrong dtype": lambda: lca.bwd_accumulate(
            q, k, v, o, lse, do, f32(q), torch.zeros_like(k), f32(v), causal=True),
        "fwd_fp8 empty descale": lambda: lca.fwd_fp8(q8, k8, v8, empty, ds[1], ds[2], causal=True),
        "bwd_fp8 lse of the wrong shape": lambda: lca.bwd_fp8(
            q8, k8, v8, *ds, torch.empty((B, S, Hq, 128), dtype=torch.bfloat16, device="cuda"), bad_lse,
            torch.empty((B, S, Hq, 128), dtype=torch.bfloat16, device="cuda"), causal=True),
    }
    for what, call in calls.items():
        print(f"case binding check: {what}", flush=True)
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
