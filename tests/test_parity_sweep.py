"""A seeded sweep of small random shapes through every bf16 entry point, against the fp64 oracle.

Each case draws batch, GQA group, kv heads, sequence length (ragged, from 1),
head dim, mask and (for batch 1) a random packing, then checks through the
C ABI:
* attn_fwd: O and LSE to the forward bar (check_fwd);
* attn_bwd: dQ, dK, dV rel-L2 <= 1e-2 (check_grads);
* attn_fwd_merge: one ring step into a random running result, against the
  oracle's merge;
* attn_bwd_accumulate (accumulate off): rounds to attn_bwd's output bit for bit.
The draws are fixed by the seed, so a failure names a reproducible case.
"""
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


CASES = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sweep_case(case):
    import torch
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D, causal, lengths = CASES[case]
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
