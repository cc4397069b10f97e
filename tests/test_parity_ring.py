"""GPU parity for the Ring-Attention pieces, through the C ABI.

* attn_merge against the oracle's merge of two partial results, including
  parts with no visible key (LSE = -inf) and rows where neither part has one;
* a ring forward on one GPU: the sequence is cut into N chunks, query chunk r
  attends to key chunks c <= r (non-causal for c < r, causal for c = r) with
  attn_fwd, and the partial results are merged in ring order. It must equal
  the oracle's full attention (bf16 tolerances: O max-abs <= 1e-2, or half a
  bf16 ulp where that is larger, rel-L2 <= 5e-3; LSE <= 1e-3);
* the matching backward: attn_bwd on every (query chunk, key chunk) pair with
  the final O and LSE gives the global probabilities restricted to that
  chunk pair, so the pair gradients summed over chunks must equal the
  oracle's full gradients (rel-L2 <= 1e-2);
* attn_fwd_merge, the forward that merges its result into the running one
  itself: one step against the oracle's merge of a random running result
  with the oracle's attention (causal or not, GQA, packed, the key split whose
  combine does the merge, accumulate off, the bf16 copy), rows with fewer
  than 64 visible keys to fp32 accuracy; and the whole ring built from it,
  forward and backward (the backward with attn_bwd_accumulate), as above;
* attn_fwd_fp8_merge, one step and an fp8 ring, against the oracle on the
  dequantised inputs;
* attn_bwd_accumulate against attn_bwd: with accumulate off its fp32 result
  rounds to attn_bwd's bf16 output bit for bit, and with accumulate on it is
  the running sum plus that result (one fp32 rounding), with and without the
  head and key splits.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import check_fwd, check_grads, dev_bf16, dev_i32, host, max_abs, rounding_o_bound

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_exact_fwd_amd as lca
    return lca


MERGE_CASES = [
    # B, S, H, D, accumulate, with_out
    (1, 37, 3, 128, True, True),
    (2, 100, 2, 64, True, False),
    (1, 1, 1, 128, False, True),
    (1, 513, 5, 64, False, False),
]


@pytest.mark.parametrize("B,S,H,D,acc,with_out", MERGE_CASES)
def test_merge_kernel_matches_oracle(B, S, H, D, acc, with_out):
    import torch
    lca = _lib()
    print(f"merge B={B} S={S} H={H} D={D} accumulate={acc} out={with_out}", flush=True)
    rng = np.random.default_rng(S * 31 + H)
    o1 = rng.standard_normal((B, S, H, D)).astype(np.float32)
    l1 = rng.uniform(-20, 20, (B, H, S)).astype(np.float32)
    p_bits = si.bf16_bits_from_f32(rng.standard_normal((B, S, H, D)).astype(np.float32))
    l2 = (l1 + rng.uniform(-30, 30, (B, H, S))).astype(np.float32)
    # empty parts: some rows with no key in the running part, some in the new part, some in both
    l1.reshape(-1)[::7] = -np.inf
    l2.reshape(-1)[::5] = -np.inf
    dev = torch.device("cuda")
    o_acc = torch.from_numpy(o1.copy()).to(dev)
    lse_acc = torch.from_numpy(l1.copy()).to(dev)
    o_part = dev_bf16(p_bits)
    lse_part = torch.from_numpy(l2).to(dev)
    o_out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev) if with_out else None
    lca.merge(o_acc, lse_acc, o_part, lse_part, accumulate=acc, o_out=o_out)
    torch.cuda.synchronize()
    r_o1 = o1.astype(np.float64) if acc else np.zeros_like(o1, dtype=np.float64)
    r_l1 = l1.astype(np.float64) if acc else np.full(l1.shape, -np.inf)
    ro, rl = oracle.merge_partials(r_o1, r_l1, si.bf16_bits_to_f64(p_bits), l2.astype(np.float64))
    go, gl = host(o_acc), host(lse_acc)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), "empty rows differ"
    fin = np.isfinite(rl)
    err_l = float(np.max(np.abs(gl[fin] - rl[fin]))) if fin.any() else 0.0
    err_o = max_abs(go, ro)
    print(f"merge O maxabs={err_o:.3e} LSE maxabs={err_l:.3e}", flush=True)
    # fp32 arithmetic on O(1) values and LSEs of magnitude <= 50
    assert err_o <= 2e-6 and err_l <= 2e-5
    if with_out:
        # the bf16 copy is the fp32 result rounded to nearest
        gb = host(o_out)
        assert np.max(np.abs(gb - go) - np.abs(go) * 2.0 ** -8) <= 0.0


def _ring_inputs(B, Hq, Hkv, S, D, seed):
    x = si.make_inputs(B, Hq, Hkv, S, D, seed)
    return x, dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)


def ring_forward(q, k, v, nchunk, causal, scale):
    """Ring order on one GPU: query chunk r merges its partials over key chunks 0..r (all chunks if not causal)."""
    import torch
    lca = _lib()
    B, S, Hq, D = q.shape
    L = S // nchunk
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    for r in range(nchunk):
        qr = q[:, r * L:(r + 1) * L].contiguous()
        o_acc = torch.empty((B, L, Hq, D), dtype=torch.float32, device=q.device)
        l_acc = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
        o_r = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=q.device)
        chunks = list(range(r + 1)) if causal else list(range(nchunk))
        for i, c in enumerate(chunks):
            kc = k[:, c * L:(c + 1) * L].contiguous()
            vc = v[:, c * L:(c + 1) * L].contiguous()
            po, pl = lca.fwd(qr, kc, vc, causal=(causal and c == r), scale=scale)
            lca.merge(o_acc, l_acc, po, pl, accumulate=(i > 0), o_out=o_r if i == len(chunks) - 1 else None)
        o[:, r * L:(r + 1) * L] = o_r
        lse[:, :, r * L:(r + 1) * L] = l_acc
    return o, lse


def ring_forward_fused(q, k, v, nchunk, causal, scale):
    """ring_forward with attn_fwd_merge: each key chunk's result goes straight into the running one."""
    import torch
    lca = _lib()
    B, S, Hq, D = q.shape
    L = S // nchunk
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    for r in range(nchunk):
        qr = q[:, r * L:(r + 1) * L].contiguous()
        o_acc = torch.empty((B, L, Hq, D), dtype=torch.float32, device=q.device)
        l_acc = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
        o_r = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device=q.device)
        chunks = list(range(r + 1)) if causal else list(range(nchunk))
        for i, c in enumerate(chunks):
            lca.fwd_merge(qr, k[:, c * L:(c + 1) * L].contiguous(), v[:, c * L:(c + 1) * L].contiguous(), o_acc,
                          l_acc, causal=(causal and c == r), accumulate=(i > 0), scale=scale,
                          o_out=o_r if i == len(chunks) - 1 else None)
        o[:, r * L:(r + 1) * L] = o_r
        lse[:, :, r * L:(r + 1) * L] = l_acc
    return o, lse


def ring_backward(q, k, v, o, lse, do, nchunk, causal, scale):
    """Pair backward with the final O and LSE; gradients summed over chunk pairs in fp32."""
    import torch
    lca = _lib()
    B, S, Hq, D = q.shape
    L = S // nchunk
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    for r in range(nchunk):
        rs = slice(r * L, (r + 1) * L)
        qr, orr, dor = q[:, rs].contiguous(), o[:, rs].contiguous(), do[:, rs].contiguous()
        lr = lse[:, :, rs].contiguous()
        for c in (range(r + 1) if causal else range(nchunk)):
            cs = slice(c * L, (c + 1) * L)
            g = lca.bwd(qr, k[:, cs].contiguous(), v[:, cs].contiguous(), orr, lr, dor,
                        causal=(causal and c == r), scale=scale)
            dq[:, rs] += g[0].float()
            dk[:, cs] += g[1].float()
            dv[:, cs] += g[2].float()
    return dq, dk, dv


def ring_backward_accumulate(q, k, v, o, lse, do, nchunk, causal, scale):
    """ring_backward with attn_bwd_accumulate: each pair's gradients are added to per-chunk fp32 sums by the
    kernels (sums start at zero; accumulate=False is covered on its own below)."""
    import torch
    lca = _lib()
    B, S, Hq, D = q.shape
    L = S // nchunk
    dq_c = [torch.zeros((B, L, Hq, D), dtype=torch.float32, device=q.device) for _ in range(nchunk)]
    dk_c = [torch.zeros((B, L) + tuple(k.shape[2:]), dtype=torch.float32, device=q.device) for _ in range(nchunk)]
    dv_c = [torch.zeros((B, L) + tuple(v.shape[2:]), dtype=torch.float32, device=q.device) for _ in range(nchunk)]
    for r in range(nchunk):
        rs = slice(r * L, (r + 1) * L)
        qr, orr, dor = q[:, rs].contiguous(), o[:, rs].contiguous(), do[:, rs].contiguous()
        lr = lse[:, :, rs].contiguous()
        for c in (range(r + 1) if causal else range(nchunk)):
            cs = slice(c * L, (c + 1) * L)
            lca.bwd_accumulate(qr, k[:, cs].contiguous(), v[:, cs].contiguous(), orr, lr, dor, dq_c[r], dk_c[c],
                               dv_c[c], causal=(causal and c == r), accumulate=True, scale=scale)
    return torch.cat(dq_c, dim=1), torch.cat(dk_c, dim=1), torch.cat(dv_c, dim=1)


RING_CASES = [
    # B, Hq, Hkv, S, D, nchunk, causal
    (1, 4, 2, 512, 128, 2, True),
    (1, 4, 2, 512, 128, 4, True),
    (2, 2, 1, 384, 64, 3, True),
    (1, 3, 3, 256, 128, 4, False),
]


@pytest.mark.parametrize("fused", [False, True], ids=["fwd+merge", "fwd_merge"])
@pytest.mark.parametrize("B,Hq,Hkv,S,D,nchunk,causal", RING_CASES)
def test_ring_forward_and_backward_equal_full_attention(B, Hq, Hkv, S, D, nchunk, causal, fused):
    import torch
    print(f"ring B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} N={nchunk} causal={causal} fused={fused}", flush=True)
    x, q, k, v, do = _ring_inputs(B, Hq, Hkv, S, D, seed=90 + nchunk)
    scale = 1.0 / np.sqrt(D)
    o, lse = (ring_forward_fused if fused else ring_forward)(q, k, v, nchunk, causal, scale)
    torch.cuda.synchronize()
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    check_fwd(host(o), host(lse), ro, rl, tag="ring fwd")
    dq, dk, dv = (ring_backward_accumulate if fused else ring_backward)(q, k, v, o, lse, do, nchunk, causal, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, x.values("do"), causal=causal, scale=scale, workers=None)
    check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)], tag="ring bwd")


FUSED_CASES = [
    # B, Hq, Hkv, S, D, causal, packed lengths, accumulate, bf16 copy, key split
    (1, 4, 2, 300, 128, True, None, True, True, False),
    (2, 2, 1, 200, 64, False, None, False, False, False),
    (1, 2, 2, 300, 128, True, [37, 63, 200], True, False, False),
    (1, 3, 1, 250, 64, False, [10, 50, 64, 126], True, True, False),
    (1, 2, 1, 4500, 128, True, None, True, True, True),
    (1, 2, 2, 4400, 64, True, [50, 4000, 350], True, False, True),
    (1, 2, 1, 4200, 128, False, None, False, True, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths,acc,with_out,split", FUSED_CASES)
def test_fwd_merge_step_matches_oracle(B, Hq, Hkv, S, D, causal, lengths, acc, with_out, split):
    import torch
    lca = _lib()
    print(f"fwd_merge B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} accumulate={acc} "
          f"out={with_out} split={split}", flush=True)
    if split:
        assert lca.fwd_workspace_bytes(B, Hq, Hkv, S, D) > 0, "case meant to run the key split"
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=S + 7 * Hq + D, lengths=lengths, with_do=False)
    rng = np.random.default_rng(S * 3 + D)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    # running LSEs around the new part's (ln of the visible key count, plus about 0.5)
    l1 = rng.uniform(-2.0, 10.0, (B, Hq, S)).astype(np.float32)
    l1.reshape(-1)[::9] = -np.inf  # rows whose running result is still empty
    dev = torch.device("cuda")
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    o_acc = torch.from_numpy(o1.copy()).to(dev)
    lse_acc = torch.from_numpy(l1.copy()).to(dev)
    o_out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev) if with_out else None
    scale = 1.0 / np.sqrt(D)
    lca.fwd_merge(q, k, v, o_acc, lse_acc, causal=causal, accumulate=acc, o_out=o_out, cu_seqlens=cu, scale=scale,
                  split=split)
    torch.cuda.synchronize()
    po, pl = oracle.attention_fwd(x.values("q"), x.values("k"), x.values("v"), causal=causal, scale=scale,
                                  cu_seqlens=x.cu_seqlens, workers=None)
    r_o1 = o1.astype(np.float64) if acc else np.zeros_like(o1, dtype=np.float64)
    r_l1 = l1.astype(np.float64) if acc else np.full(l1.shape, -np.inf)
    ro, rl = oracle.merge_partials(r_o1, r_l1, po, pl)
    go, gl = host(o_acc), host(lse_acc)
    check_fwd(go, gl, ro, rl, tag="fwd_merge")
    # rows with fewer than 64 visible keys: exact fp32 partial and fp32 merge
    s0, s1 = oracle.segment_bounds(S, x.cu_seqlens)
    pos = np.arange(S)
    few = ((pos + 1 if causal else s1) - s0) < 64
    if few.any():
        e_o = max_abs(go[:, few], ro[:, few])
        e_l = max_abs(gl[:, :, few], rl[:, :, few])
        print(f"fwd_merge few-key rows: {int(few.sum())} O maxabs={e_o:.3e} LSE maxabs={e_l:.3e}", flush=True)
        assert e_o <= 1e-5 and e_l <= 1e-5
    if with_out:
        gb = host(o_out)
        assert np.max(np.abs(gb - go) - np.abs(go) * 2.0 ** -8) <= 0.0


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", [
    (1, 4, 2, 700, 128, True, None),
    (2, 3, 1, 333, 64, False, None),
    (1, 2, 2, 600, 128, True, [100, 37, 463]),
])
def test_fwd_merge_block_geometries(B, Hq, Hkv, S, D, causal, lengths, monkeypatch):
    """attn_fwd_merge with 128-query blocks (4 waves) and 256-query blocks (8 waves): both meet the oracle bar
    and give bitwise the same running result (each row is computed and merged in the same order)."""
    import torch
    lca = _lib()
    print(f"fwd_merge geometry B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=S + D, lengths=lengths, with_do=False)
    rng = np.random.default_rng(S + 1)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l1 = rng.uniform(-2.0, 8.0, (B, Hq, S)).astype(np.float32)
    dev = torch.device("cuda")
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    po, pl = oracle.attention_fwd(x.values("q"), x.values("k"), x.values("v"), causal=causal, scale=scale,
                                  cu_seqlens=x.cu_seqlens, workers=None)
    ro, rl = oracle.merge_partials(o1.astype(np.float64), l1.astype(np.float64), po, pl)
    outs = []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        o_acc = torch.from_numpy(o1.copy()).to(dev)
        lse_acc = torch.from_numpy(l1.copy()).to(dev)
        o_out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev)
        lca.fwd_merge(q, k, v, o_acc, lse_acc, causal=causal, accumulate=True, o_out=o_out, cu_seqlens=cu,
                      scale=scale, split=False)
        torch.cuda.synchronize()
        check_fwd(host(o_acc), host(lse_acc), ro, rl, tag=f"fwd_merge waves={waves}")
        outs.append((o_acc, lse_acc, o_out))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


FP8_MERGE_CASES = [
    # B, Hq, Hkv, S, causal, packed lengths, accumulate, bf16 copy, key split
    (1, 4, 2, 300, True, None, True, True, False),
    (2, 2, 1, 200, False, None, False, False, False),
    (1, 2, 2, 300, True, [37, 63, 200], True, False, False),
    (1, 2, 1, 4500, True, None, True, True, True),
    (1, 2, 2, 4400, False, [50, 4000, 350], True, False, True),
]


def _fp8_dev(x):
    import torch
    from tests.gpu_helpers import dev_u8
    q8, k8, v8 = dev_u8(x.q_bits), dev_u8(x.k_bits), dev_u8(x.v_bits)
    ds = [torch.tensor([float(d)], dtype=torch.float32, device="cuda") for d in x.descale]
    deq = [oracle.e4m3_decode(b) * float(d) for b, d in zip((x.q_bits, x.k_bits, x.v_bits), x.descale)]
    return (q8, k8, v8), ds, deq


@pytest.mark.parametrize("B,Hq,Hkv,S,causal,lengths,acc,with_out,split", FP8_MERGE_CASES)
def test_fwd_fp8_merge_step_matches_oracle(B, Hq, Hkv, S, causal, lengths, acc, with_out, split):
    """attn_fwd_fp8_merge against the oracle's merge of a random running result with the oracle's attention over
    the dequantised inputs: O rel-L2 <= 5e-2 (the fp8 bound), LSE max-abs <= 1e-3."""
    import torch
    from tests.gpu_helpers import TOL_FP8_REL, TOL_LSE, rel_l2
    lca = _lib()
    D = 128
    print(f"fwd_fp8_merge B={B} Hq={Hq} Hkv={Hkv} S={S} causal={causal} lengths={lengths} accumulate={acc} "
          f"out={with_out} split={split}", flush=True)
    if split:
        assert lca.fwd_workspace_bytes(B, Hq, Hkv, S, D) > 0, "case meant to run the key split"
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=S + 11, lengths=lengths, fp8=True, with_do=False)
    (q8, k8, v8), ds, (qv, kv, vv) = _fp8_dev(x)
    rng = np.random.default_rng(S * 5 + 1)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l1 = rng.uniform(-2.0, 10.0, (B, Hq, S)).astype(np.float32)
    l1.reshape(-1)[::9] = -np.inf
    dev = torch.device("cuda")
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    o_acc = torch.from_numpy(o1.copy()).to(dev)
    lse_acc = torch.from_numpy(l1.copy()).to(dev)
    o_out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=dev) if with_out else None
    scale = 1.0 / np.sqrt(D)
    lca.fwd_fp8_merge(q8, k8, v8, *ds, o_acc, lse_acc, causal=causal, accumulate=acc, o_out=o_out, cu_seqlens=cu,
                      scale=scale, split=split)
    torch.cuda.synchronize()
    po, pl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    r_o1 = o1.astype(np.float64) if acc else np.zeros_like(o1, dtype=np.float64)
    r_l1 = l1.astype(np.float64) if acc else np.full(l1.shape, -np.inf)
    ro, rl = oracle.merge_partials(r_o1, r_l1, po, pl)
    go, gl = host(o_acc), host(lse_acc)
    rr, el = rel_l2(go, ro), max_abs(gl, rl)
    print(f"fwd_fp8_merge O relL2={rr:.3e} LSE maxabs={el:.3e}", flush=True)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert rr <= TOL_FP8_REL and el <= TOL_LSE
    if with_out:
        gb = host(o_out)
        assert np.max(np.abs(gb - go) - np.abs(go) * 2.0 ** -8) <= 0.0


@pytest.mark.parametrize("B,Hq,Hkv,S,nchunk,causal", [(1, 4, 2, 512, 4, True), (1, 3, 3, 384, 3, False)])
def test_fp8_ring_forward_equals_full_attention(B, Hq, Hkv, S, nchunk, causal):
    """A ring of attn_fwd_fp8_merge calls over the chunks equals the oracle's full attention on the dequantised
    inputs (fp8 bounds)."""
    import torch
    from tests.gpu_helpers import TOL_FP8_REL, TOL_LSE, rel_l2
    lca = _lib()
    D = 128
    print(f"fp8 ring B={B} Hq={Hq} Hkv={Hkv} S={S} N={nchunk} causal={causal}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=70 + nchunk, fp8=True, with_do=False)
    (q8, k8, v8), ds, (qv, kv, vv) = _fp8_dev(x)
    scale = 1.0 / np.sqrt(D)
    L = S // nchunk
    o = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    for r in range(nchunk):
        qr = q8[:, r * L:(r + 1) * L].contiguous()
        o_acc = torch.empty((B, L, Hq, D), dtype=torch.float32, device="cuda")
        l_acc = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
        o_r = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device="cuda")
        chunks = list(range(r + 1)) if causal else list(range(nchunk))
        for i, c in enumerate(chunks):
            lca.fwd_fp8_merge(qr, k8[:, c * L:(c + 1) * L].contiguous(), v8[:, c * L:(c + 1) * L].contiguous(), *ds,
                              o_acc, l_acc, causal=(causal and c == r), accumulate=(i > 0), scale=scale,
                              o_out=o_r if i == len(chunks) - 1 else None)
        o[:, r * L:(r + 1) * L] = o_r
        lse[:, :, r * L:(r + 1) * L] = l_acc
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    rr, el = rel_l2(host(o), ro), max_abs(host(lse), rl)
    print(f"fp8 ring O relL2={rr:.3e} LSE maxabs={el:.3e}", flush=True)
    assert rr <= TOL_FP8_REL and el <= TOL_LSE


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", [
    (1, 4, 2, 300, 128, True, None),           # both splits (partials + reduce kernels)
    (2, 3, 1, 200, 64, False, None),
    (1, 2, 2, 500, 128, True, [120, 380]),
    (8, 8, 8, 2048, 128, True, None),          # no split: the kernels' own epilogues
])
def test_bwd_accumulate_matches_bwd(B, Hq, Hkv, S, D, causal, lengths):
    import torch
    lca = _lib()
    print(f"bwd_accumulate B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=S + 3, lengths=lengths)
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    ref = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    acc = [torch.full(t.shape, float("nan"), dtype=torch.float32, device=t.device) for t in ref]
    lca.bwd_accumulate(q, k, v, o, lse, do, *acc, causal=causal, accumulate=False, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    for a, r, name in zip(acc, ref, ("dQ", "dK", "dV")):
        assert torch.equal(a.to(torch.bfloat16), r), f"{name}: accumulate=False does not round to attn_bwd's output"
    g = torch.Generator(device="cpu").manual_seed(S)
    init = [torch.randn(t.shape, generator=g).to(t.device) for t in acc]
    run = [t.clone() for t in init]
    lca.bwd_accumulate(q, k, v, o, lse, do, *run, causal=causal, accumulate=True, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    for a, i0, r0, name in zip(run, init, acc, ("dQ", "dK", "dV")):
        want = i0 + r0
        bound = (i0.abs() + r0.abs()) * 2.0 ** -23 + 1e-30
        excess = float(((a - want).abs() - bound).max())
        print(f"{name} accumulate=True max excess over one fp32 rounding {excess:.3e}", flush=True)
        assert excess <= 0.0, name


@pytest.mark.parametrize("qk_std,lse_span", [(1.0, 100.0), (3.0, 30.0)])
def test_fwd_merge_extreme_weights(qk_std, lse_span):
    """attn_fwd_merge where the running LSE is far above or below the new part's (weights that underflow to 0 on
    either side) and, with Q and K scaled by 3, peaky rows that take the tiled kernel's lazy rescale before the
    merge. Bars as the other forward tests (for the scaled inputs O within the bound of the kernel's rounding,
    as in the forward stress test)."""
    import torch
    lca = _lib()
    B, Hq, Hkv, S, D = 1, 4, 2, 700, 128
    print(f"fwd_merge extreme qk_std={qk_std} lse_span={lse_span}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed=77, with_do=False, qk_std=qk_std)
    rng = np.random.default_rng(78)
    o1 = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    l1 = rng.uniform(-lse_span, lse_span, (B, Hq, S)).astype(np.float32)
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    o_acc, l_acc = torch.from_numpy(o1.copy()).cuda(), torch.from_numpy(l1.copy()).cuda()
    scale = 1.0 / np.sqrt(D)
    lca.fwd_merge(q, k, v, o_acc, l_acc, causal=True, accumulate=True, scale=scale)
    torch.cuda.synchronize()
    po, pl = oracle.attention_fwd(x.values("q"), x.values("k"), x.values("v"), causal=True, scale=scale, workers=None)
    ro, rl = oracle.merge_partials(o1.astype(np.float64), l1.astype(np.float64), po, pl)
    bound = None
    if qk_std != 1.0:
        # the part's P rounding enters with the part's merge weight (at most 1); o_acc is not rounded to bf16
        abar, _ = oracle.attention_fwd(x.values("q"), x.values("k"), np.abs(x.values("v")), causal=True, scale=scale,
                                       workers=None)
        bound = rounding_o_bound(host(o_acc), ro, abar)
    check_fwd(host(o_acc), host(l_acc), ro, rl, tag="fwd_merge extreme", bound=bound)


def test_few_key_delta_only_where_the_call_holds_the_whole_row():
    """The Delta phase's two branches, read back from the workspace (its first fp32 array, [B, Hq, S64]).

    A full call: rows 0..62 (fewer than 64 visible keys) hold sum_j P_ij dP_ij, which equals dO_i . O_i for the
    exact O, so they match the oracle's Delta to fp32 rounding; later rows hold dO_i . O_i of the bf16 O the call
    was given. A ring's diagonal chunk pair past the first chunk, called with the whole rows' O and LSE: the
    call's keys carry only part of each row's P, so every row, its first 63 included, keeps dO . O of the given
    O. The first chunk's diagonal pair holds whole rows and takes the sum again."""
    import torch
    lca = _lib()
    B, Hq, Hkv, S, D, L = 1, 4, 2, 256, 128, 128
    print(f"few-key Delta branches B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} chunk={L}", flush=True)
    x, q, k, v, do = _ring_inputs(B, Hq, Hkv, S, D, seed=97)
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
    ro, _ = oracle.attention_fwd(qv, kv, vv, causal=True, scale=scale, workers=None)
    exact = np.einsum("bshd,bshd->bhs", dov, ro)                       # sum_j P_ij dP_ij
    given = np.einsum("bshd,bshd->bhs", dov, host(o))                  # dO . O with the bf16 O
    mag = np.einsum("bshd,bshd->bhs", np.abs(dov), np.abs(host(o)))   # scale of the fp32 rounding

    def delta_of(a, b, causal_call):
        n = b - a
        ws = torch.empty(lca.bwd_workspace_bytes(B, Hq, Hkv, n, D) // 4 + 1, dtype=torch.float32, device="cuda")
        sl = slice(a, b)
        lca.bwd(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(), o[:, sl].contiguous(),
                lse[:, :, sl].contiguous(), do[:, sl].contiguous(), causal=causal_call, scale=scale, workspace=ws,
                phases=lca.BWD_DELTA)
        torch.cuda.synchronize()
        s64 = (n + 63) // 64 * 64
        return ws[:B * Hq * s64].view(B, Hq, s64)[..., :n].double().cpu().numpy()

    tol = 2.0 ** -18 * (mag + 1.0)
    full = delta_of(0, S, True)
    assert np.all(np.abs(full[..., :63] - exact[..., :63]) <= tol[..., :63]), "full call: rows 0..62 are not the sum"
    assert np.all(np.abs(full[..., 63:] - given[..., 63:]) <= tol[..., 63:]), "full call: rows 63.. are not dO . O"
    first = delta_of(0, L, True)
    assert np.all(np.abs(first[..., :63] - exact[..., :63]) <= tol[..., :63]), "first chunk: rows 0..62"
    pair = delta_of(L, 2 * L, True)
    assert np.all(np.abs(pair - given[..., L:]) <= tol[..., L:]), "later diagonal chunk: Delta is not dO . O"
    # the two branches differ here, so the checks above tell them apart
    gap = float(np.max(np.abs(exact[..., :63] - given[..., :63]) / tol[..., :63]))
    print(f"few-key Delta: largest |sum - dO.O| over the first 63 rows = {gap:.1f} x the fp32 tolerance", flush=True)
    assert gap > 4.0
