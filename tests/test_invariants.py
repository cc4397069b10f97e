"""GPU: identities the exact computation must satisfy, checked on whole outputs
of the full-size workloads without the oracle.

- Ulysses head share ("ms-swift长文本训练秘诀：Ulysses并行技术解析", the
  equivalence of the split and unsplit computation): running only a share of
  the heads (Hq/2 query heads with their Hkv/2 kv heads) gives those heads'
  results of the full run. Forward and dQ do the same arithmetic in the same
  order, so they agree bitwise; dK/dV of the smaller grid split the group's
  heads differently (another fp32 summation order), so they agree up to
  rounding.
- GQA as MHA: a GQA run equals an MHA run on K and V repeated over each
  group (forward and dQ bitwise; the group's dK/dV are the sums of the MHA
  heads' dK/dV, up to the bf16 rounding of each term).
- Packing (the packing of the Ulysses page §5): a packed run equals the
  concatenation of runs on each segment alone, up to rounding: the tiles of
  a segment start at different offsets, so sums are ordered differently and
  the running maximum, hence the bf16 rounding of P, can differ.
- The first row of a causal segment sees one key: O is that key's V row
  exactly and LSE is the scaled score.

"Up to rounding" is checked as: for the head shares, dK/dV rel-L2 <= 1e-3
(an order of magnitude inside the oracle bar); for GQA against MHA every
dK/dV element within the bf16 rounding of the terms of its group sum; for
packing, O within the oracle's O bar (rel-L2 <= 5e-3, 1e-2 per element) and
LSE within 1e-5, because the two runs round P to bf16 against different
running maxima and so differ by about the kernel's own error (measured up to
1.5e-3), and the gradients, which see that O through Delta, rel-L2 <= 5e-3.
"""
import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu


def _lca():
    import long_context_exact_fwd_amd as lca
    return lca


def _inputs(x):
    lca = _lca()
    q, k, v = (lca.bf16_from_bits(b, "cuda") for b in (x.q_bits, x.k_bits, x.v_bits))
    do = lca.bf16_from_bits(x.do_bits, "cuda") if x.do_bits is not None else None
    return q, k, v, do


def _run(q, k, v, do, causal, cu=None, scale=None):
    lca = _lca()
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    return o, lse, dq, dk, dv


def _ulp(x):
    """Spacing of bfloat16 values at |x| (x float or double)."""
    import torch
    return torch.exp2(torch.floor(torch.log2(x.abs().clamp_min(2.0 ** -126))) - 7.0)


def _rel_l2(a, b, what, tol=1e-3):
    import torch
    a64, b64 = a.double(), b.double()
    e = float(torch.linalg.vector_norm(a64 - b64) / torch.linalg.vector_norm(b64))
    print(f"{what}: relL2 {e:.3e}", flush=True)
    assert e <= tol, what


def test_ulysses_head_share_equals_the_full_run():
    """gqa32k (Hq 28, Hkv 4) against its two 2-way Ulysses shares (Hq 14, Hkv 2 each)."""
    import torch
    w = si.WORKLOADS["gqa32k"]
    print("invariant: Ulysses head shares of gqa32k", flush=True)
    q, k, v, do = _inputs(si.workload_inputs(w, with_do=True))
    full = _run(q, k, v, do, w.causal, scale=w.scale)
    torch.cuda.synchronize()
    hq, hkv = w.hq // 2, w.hkv // 2
    for r in range(2):
        qs, dos = (t[:, :, r * hq:(r + 1) * hq].contiguous() for t in (q, do))
        ks, vs = (t[:, :, r * hkv:(r + 1) * hkv].contiguous() for t in (k, v))
        o, lse, dq, dk, dv = _run(qs, ks, vs, dos, w.causal, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, full[0][:, :, r * hq:(r + 1) * hq]), f"share {r}: O"
        assert torch.equal(lse, full[1][:, r * hq:(r + 1) * hq]), f"share {r}: LSE"
        assert torch.equal(dq, full[2][:, :, r * hq:(r + 1) * hq]), f"share {r}: dQ"
        _rel_l2(dk, full[3][:, :, r * hkv:(r + 1) * hkv], f"share {r}: dK")
        _rel_l2(dv, full[4][:, :, r * hkv:(r + 1) * hkv], f"share {r}: dV")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [(1, 8, 2, 4096, 128, True), (2, 6, 3, 3000, 64, False)])
def test_gqa_equals_mha_on_repeated_kv(B, Hq, Hkv, S, D, causal):
    import torch
    print(f"invariant: GQA as MHA B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal}", flush=True)
    q, k, v, do = _inputs(si.make_inputs(B, Hq, Hkv, S, D, 73, with_do=True))
    G = Hq // Hkv
    gqa = _run(q, k, v, do, causal)
    kr, vr = (t.repeat_interleave(G, dim=2).contiguous() for t in (k, v))
    mha = _run(q, kr, vr, do, causal)
    torch.cuda.synchronize()
    assert torch.equal(gqa[0], mha[0]) and torch.equal(gqa[1], mha[1]) and torch.equal(gqa[2], mha[2])
    for i, name in ((3, "dK"), (4, "dV")):
        # GQA rounds the fp32 group sum once; the MHA heads round each term: the two differ by at most half
        # an ulp of the GQA value plus half an ulp of every MHA term (and fp32 noise far below that)
        terms = mha[i].double().reshape(B, S, Hkv, G, D)
        g = gqa[i].double()
        bound = 0.5 * _ulp(g) + 0.5 * _ulp(terms).sum(dim=3) + 2.0 ** -20 * terms.abs().sum(dim=3) + 1e-8
        worst = float(((g - terms.sum(dim=3)).abs() / bound).max())
        print(f"GQA {name} vs summed MHA {name}: worst {worst:.2f} of the rounding bound", flush=True)
        assert worst <= 1.0, name


def test_packed_run_equals_per_segment_runs():
    """packed32k against each of its five segments run as an unpacked sequence."""
    import torch
    w = si.WORKLOADS["packed32k"]
    print("invariant: packed32k against its segments", flush=True)
    x = si.workload_inputs(w, with_do=True)
    q, k, v, do = _inputs(x)
    cu = torch.from_numpy(x.cu_seqlens).to("cuda")
    packed = _run(q, k, v, do, w.causal, cu=cu, scale=w.scale)
    torch.cuda.synchronize()
    bounds = [(int(a), int(b)) for a, b in zip(x.cu_seqlens[:-1], x.cu_seqlens[1:])]
    for a, b in bounds:
        seg = [t[:, a:b].contiguous() for t in (q, k, v, do)]
        o, lse, dq, dk, dv = _run(*seg, w.causal, scale=w.scale)
        torch.cuda.synchronize()
        _rel_l2(o, packed[0][:, a:b], f"segment [{a}, {b}): O", tol=5e-3)
        o_diff = float((o.float() - packed[0][:, a:b].float()).abs().max())
        assert o_diff <= 1e-2, f"segment [{a}, {b}): O max diff {o_diff}"
        lse_diff = float((lse - packed[1][:, :, a:b]).abs().max())
        print(f"segment [{a}, {b}): LSE max diff {lse_diff:.2e}", flush=True)
        assert lse_diff <= 1e-5
        for got, ref, name in ((dq, packed[2][:, a:b], "dQ"), (dk, packed[3][:, a:b], "dK"),
                               (dv, packed[4][:, a:b], "dV")):
            _rel_l2(got, ref, f"segment [{a}, {b}): {name}", tol=5e-3)


def test_first_row_of_each_causal_segment_is_its_value_row():
    import torch
    lca = _lca()
    w = si.WORKLOADS["packed32k"]
    print("invariant: first rows of the packed32k segments", flush=True)
    x = si.workload_inputs(w, with_do=False)
    q, k, v, _ = _inputs(x)
    cu = torch.from_numpy(x.cu_seqlens).to("cuda")
    o, lse = lca.fwd(q, k, v, causal=True, cu_seqlens=cu, scale=w.scale)
    torch.cuda.synchronize()
    G = w.hq // w.hkv
    qv, kv = x.values("q"), x.values("k")
    lse_h = lse.cpu().numpy()
    for s0 in x.cu_seqlens[:-1]:
        s0 = int(s0)
        for h in range(w.hq):
            assert torch.equal(o[0, s0, h], v[0, s0, h // G]), f"row {s0} head {h}"
            ref = w.scale * float(np.dot(qv[0, s0, h], kv[0, s0, h // G]))
            assert abs(float(lse_h[0, h, s0]) - ref) <= 1e-4 * max(1.0, abs(ref)), f"LSE row {s0} head {h}"
