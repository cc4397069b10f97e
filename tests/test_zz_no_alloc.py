"""attn_bwd_noalloc (the backward with the library's fixed scratch instead of a
caller workspace) against attn_bwd, through the C ABI.

Two calls in a row, the second on a smaller input, so the second runs on
scratch that still holds the first call's contents. Both shapes fit the
scratch with attn_bwd's own splits, so the results must be bitwise equal to
attn_bwd's. A third shape needs more than the scratch for its split partials:
the backward then runs unsplit, and must still meet the gradient bar
(rel-L2 <= 1e-2) against attn_bwd and against the fp64 oracle on sampled rows.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import TOL_GRAD_REL, dev_bf16, dev_i32, host, rel_l2

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, S, D, seed, lengths=None):
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, with_do=True)
    t = [dev_bf16(b) for b in (x.q_bits, x.k_bits, x.v_bits, x.do_bits)]
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    return x, t, cu


def test_noalloc_matches_bwd_on_two_calls_in_a_row():
    import torch
    import long_context_exact_fwd_amd as lca
    for (B, Hq, Hkv, S, D, causal, lengths, seed) in [(1, 8, 2, 2048, 128, True, [700, 1, 1347], 61),
                                                      (2, 3, 1, 333, 64, False, None, 62)]:
        print(f"noalloc case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
        assert lca.bwd_workspace_bytes(B, Hq, Hkv, S, D) <= lca.NOALLOC_SCRATCH_BYTES
        x, (q, k, v, do), cu = _inputs(B, Hq, Hkv, S, D, seed, lengths)
        kw = dict(causal=causal, cu_seqlens=cu, scale=1.0 / np.sqrt(D))
        o, lse = lca.fwd(q, k, v, **kw)
        ref = lca.bwd(q, k, v, o, lse, do, **kw)
        torch.cuda.synchronize()
        got = lca.bwd_noalloc(q, k, v, o, lse, do, **kw)
        torch.cuda.synchronize()
        for name, a, r in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, r), name
        print("noalloc: bitwise equal to attn_bwd", flush=True)


def test_noalloc_runs_unsplit_when_the_partials_do_not_fit():
    import torch
    import long_context_exact_fwd_amd as lca
    B, Hq, Hkv, S, D = 1, 2, 1, 16384, 128  # attn_bwd splits heads and key tiles: 2 * 64 MiB + 32 MiB partials
    print(f"noalloc unsplit case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal", flush=True)
    assert lca.bwd_workspace_bytes(B, Hq, Hkv, S, D) > lca.NOALLOC_SCRATCH_BYTES
    x, (q, k, v, do), _ = _inputs(B, Hq, Hkv, S, D, 63)
    kw = dict(causal=True, scale=1.0 / np.sqrt(D))
    o, lse = lca.fwd(q, k, v, **kw)
    ref = [host(t) for t in lca.bwd(q, k, v, o, lse, do, **kw)]
    got = [host(t) for t in lca.bwd_noalloc(q, k, v, o, lse, do, **kw)]
    torch.cuda.synchronize()
    errs = [rel_l2(a, r) for a, r in zip(got, ref)]
    print(f"noalloc unsplit vs attn_bwd: dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
    assert max(errs) <= TOL_GRAD_REL
    rows = si.sample_indices(63, S, 24, must=[0, 1, S - 1])
    picks = [(0, h, int(i)) for h in range(Hq) for i in rows]
    qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
    rq = oracle.attention_dq_rows(qv, kv, vv, dov, picks, causal=True, scale=kw["scale"])
    e_q = rel_l2(np.stack([got[0][0, i, h] for _, h, i in picks]), rq)
    kpicks = [(0, 0, int(j)) for j in rows]
    rk, rv = oracle.attention_dkdv_rows(qv, kv, vv, dov, kpicks, causal=True, scale=kw["scale"])
    e_k = rel_l2(np.stack([got[1][0, j, 0] for _, _, j in kpicks]), rk)
    e_v = rel_l2(np.stack([got[2][0, j, 0] for _, _, j in kpicks]), rv)
    print(f"noalloc unsplit vs oracle: dQ {e_q:.3e} dK {e_k:.3e} dV {e_v:.3e}", flush=True)
    assert max(e_q, e_k, e_v) <= TOL_GRAD_REL
