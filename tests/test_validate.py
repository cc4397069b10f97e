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
