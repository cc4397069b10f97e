"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle,
element by element, on shapes the oracle finishes in seconds. They span
several tiles and ragged tails, GQA groups, packed segments and both masks.

Tolerances (from the fp64 oracle): O max-abs <= 1e-2 and rel-L2 <= 5e-3,
LSE max-abs <= 1e-3, dQ/dK/dV rel-L2 <= 1e-2 each.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_helpers import (TOL_GRAD_REL, check_fwd, check_grads, delta_from_o_rows, dev_bf16, dev_i32, host,
                               rel_l2, rounding_o_bound)

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_exact_fwd_amd as lca
    return lca


def _stress_bound(o, ro, qv, kv, vv, causal, scale, cu_seqlens=None):
    """rounding_o_bound with the attention of the same scores over |V| from the oracle."""
    abar, _ = oracle.attention_fwd(qv, kv, np.abs(vv), causal=causal, scale=scale, cu_seqlens=cu_seqlens,
                                   workers=None)
    return rounding_o_bound(o, ro, abar)


def _run_case(B, Hq, Hkv, S, D, causal, lengths=None, seed=11, backward=True, qk_std=1.0, stress=False):
    import torch
    lca = _lib()
    print(f"case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} seed={seed}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, with_do=backward, qk_std=qk_std)
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens, workers=None)
    bound = _stress_bound(host(o), ro, qv, kv, vv, causal, scale, x.cu_seqlens) if stress else None
    check_fwd(host(o), host(lse), ro, rl, tag="fwd", bound=bound)
    if not backward:
        return
    do = dev_bf16(x.do_bits)
    dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, x.values("do"), causal=causal, scale=scale,
                                      cu_seqlens=x.cu_seqlens, workers=None)
    check_grads([("dQ", host(dq), rq), ("dK", host(dk), rk), ("dV", host(dv), rv)], tag="bwd")


@pytest.mark.parametrize("causal", [True, False])
def test_tiny_workload(causal):
    """B=1, H=2, S=256, D=64, seed 1: fwd + bwd, both masks, whole tensors."""
    w = si.WORKLOADS["tiny"]
    _run_case(w.batch, w.hq, w.hkv, w.seqlen, w.head_dim, causal, seed=w.seed)


def _short_segments(seed, total, hi):
    """Seeded segment lengths in [1, hi] summing to total (the last one takes the remainder)."""
    rng = np.random.default_rng(seed)
    out = []
    while sum(out) < total:
        out.append(int(min(rng.integers(1, hi + 1), total - sum(out))))
    return out


EDGE = [
    # B, Hq, Hkv, S, D, causal, lengths
    (1, 1, 1, 1, 64, True, None),
    (1, 2, 1, 1, 128, False, None),
    (2, 2, 2, 17, 64, True, None),
    (1, 4, 2, 17, 128, False, None),
    (2, 3, 1, 100, 128, True, None),
    (1, 7, 1, 100, 64, False, None),
    (1, 2, 2, 1000, 128, True, None),
    (1, 8, 1, 1000, 128, False, None),
    (2, 4, 4, 333, 64, True, None),
    (1, 2, 1, 256, 128, True, [1, 16, 239]),
    (1, 4, 2, 256, 64, False, [1, 16, 239]),
    (1, 7, 1, 1000, 128, True, [100, 1, 1, 64, 65, 500, 269]),
    (1, 2, 2, 700, 128, False, [300, 400]),
    (1, 14, 2, 2048, 128, True, None),
    (1, 2, 1, 64, 128, True, [1] * 64),           # every segment one token: O = V, LSE = scale q.k
    (1, 3, 3, 80, 64, False, [1] * 80),
    (1, 3, 3, 320, 64, False, [64, 64, 128, 64]),  # segments ending on tile boundaries
    # about 150 short segments straddling tiles: nearly every row a few-key row
    (1, 4, 2, 3000, 128, True, _short_segments(91, 3000, 40)),
    (1, 2, 1, 2500, 64, False, _short_segments(92, 2500, 90)),  # both sides of 64 keys, non-causal
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", EDGE)
def test_edge_shapes(B, Hq, Hkv, S, D, causal, lengths):
    _run_case(B, Hq, Hkv, S, D, causal, lengths=lengths)


def test_packed_random_lengths_gqa():
    """Packed Ulysses-share shape at reduced length: seeded lengths in [64, 1024] summing to 4096."""
    rng = np.random.default_rng(44)
    lengths = si.packed_lengths(rng, total=4096, lo=64, hi=1024)
    _run_case(1, 14, 2, 4096, 128, True, lengths=lengths, seed=45)


def test_peaky_scores_exercise_rescaling():
    """Q and K scaled by 3 (score std ~9): the running maximum moves often, the lazy rescale path runs.

    Stress input outside the stated workloads: with a few dominant keys the bf16 rounding of P (up to 2^-8
    relative) does not average out, so O is held to the bound of the kernel's rounding, rounding_o_bound
    (2^-8 times the attention over |V|, plus half an ulp of the output), instead of 1e-2; rel-L2, LSE and
    gradient bounds are unchanged.
    """
    _run_case(1, 4, 1, 1500, 128, True, seed=46, qk_std=3.0, stress=True)


def _given_o_gradients(qv, kv, vv, dov, o_given, causal, scale):
    """The oracle's gradients for a backward given O in bf16, as the C ABI passes it.

    The backward uses Delta_i = dO_i . O_i with the O it is given, in the rows that see at least 64 keys
    (delta_from_o_rows; the others take Delta from its definition). Delta enters dS_ij = P_ij (dP_ij - Delta_i)
    linearly, so with eps_i = dO_i . (O_given - O)_i in those rows (0 in the others) the gradients are the
    exact ones minus scale eps_i sum_j P_ij K_j for dQ (the oracle's forward with V := K) and minus
    scale sum_i P_ij eps_i Q_i for dK (the dV of the oracle's backward with dO := eps Q); dV does not
    depend on Delta. Rows whose softmax is dominated by one key make dP - Delta a small difference,
    and this is where the bf16 rounding of O shows: with one outlier channel it moves dQ by ~2e-2."""
    ro, _ = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    rq, rk, rv = oracle.attention_bwd(qv, kv, vv, dov, causal=causal, scale=scale, workers=None)
    eps = np.einsum("bshd,bshd->bsh", dov, np.asarray(o_given, dtype=np.float64) - ro)[..., None]
    eps *= delta_from_o_rows(qv.shape[1], causal)[None, :, None, None]
    kbar, _ = oracle.attention_fwd(qv, kv, kv, causal=causal, scale=scale, workers=None)
    _, _, corr = oracle.attention_bwd(qv, kv, vv, eps * qv, causal=causal, scale=scale, workers=None)
    return rq - scale * eps * kbar, rk - scale * corr, rv, eps


def _run_bits(B, Hq, Hkv, S, D, causal, x, tag, stress=False):
    """Forward against the oracle, and the backward against the oracle's gradients given the kernel's
    own bf16 O (_given_o_gradients), on the inputs held in x (bf16 bit patterns)."""
    import torch
    lca = _lib()
    q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
    scale = 1.0 / np.sqrt(D)
    o, lse = lca.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    bound = _stress_bound(host(o), ro, qv, kv, vv, causal, scale) if stress else None
    check_fwd(host(o), host(lse), ro, rl, tag=f"{tag} fwd", bound=bound)
    rq, rk, rv, eps = _given_o_gradients(qv, kv, vv, dov, host(o), causal, scale)
    return host(o), (host(dq), host(dk), host(dv)), (rq, rk, rv), (qv, kv, vv, dov, eps, scale)


@pytest.mark.parametrize("causal", [True, False])
def test_all_equal_keys_give_the_mean_of_the_visible_values(causal):
    """Every key row the same vector: each row's softmax is uniform over its visible keys, so O is the
    mean of those V rows (checked against the oracle and the running means), and dQ = scale K sum_j dS_ij
    is zero exactly. The kernel's dQ is then the rounding of dS to bf16 plus the given-O term: each row
    within scale max|K| (|eps_i| + 2^-8 |dO_i| max_j |V_j|), since sum_j |dS_ij| <= 2 |dO_i| max_j |V_j|."""
    B, Hq, Hkv, S, D = 1, 4, 2, 700, 128
    print(f"case all-equal keys causal={causal}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 47, with_do=True)
    x.k_bits = np.ascontiguousarray(np.broadcast_to(x.k_bits[:, :1], x.k_bits.shape))
    o, got, ref, (qv, kv, vv, dov, eps, scale) = _run_bits(B, Hq, Hkv, S, D, causal, x,
                                                           f"all-equal keys causal={causal}")
    check_grads([("dK", got[1], ref[1]), ("dV", got[2], ref[2])], tag=f"all-equal keys causal={causal} bwd")
    G = Hq // Hkv
    vmax = float(np.max(np.linalg.norm(vv, axis=-1)))
    bound = scale * float(np.max(np.abs(kv))) * (np.abs(eps) + 2.0 ** -8 * np.linalg.norm(dov, axis=-1,
                                                                                       keepdims=True) * vmax)
    worst = float(np.max(np.abs(got[0] - ref[0]) / bound))
    print(f"all-equal keys dQ: max |dQ| = {np.max(np.abs(got[0])):.2e}, worst {worst:.3f} of the bound", flush=True)
    assert np.all(np.isfinite(got[0])) and worst <= 1.0
    for h in (0, Hq - 1):
        vh = vv[0, :, h // G]
        mean = np.cumsum(vh, axis=0) / np.arange(1, S + 1)[:, None] if causal else np.broadcast_to(vh.mean(0), vh.shape)
        err = float(np.max(np.abs(o[0, :, h] - mean)))
        print(f"head {h}: max |O - mean of visible V| = {err:.2e}", flush=True)
        assert err <= 1e-2


def test_one_outlier_channel_dominates_the_scores():
    """Channel 0 of Q and K scaled by 16: the scores are dominated by one product per pair (a common
    activation outlier), their spread is large and the running maximum moves. O is held to the bound of
    the kernel's rounding, as in the peaky case; the gradients meet the usual 1e-2 against the oracle's
    gradients given the kernel's bf16 O."""
    B, Hq, Hkv, S, D = 1, 4, 1, 1200, 64
    print("case outlier channel", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 51, with_do=True)
    for name in ("q_bits", "k_bits"):
        vals = si.bf16_bits_to_f64(getattr(x, name))
        vals[..., 0] *= 16.0  # a power of two: still exactly bf16
        setattr(x, name, si.bf16_bits_from_f32(vals.astype(np.float32)))
    _, got, ref, _ = _run_bits(B, Hq, Hkv, S, D, True, x, "outlier channel", stress=True)
    check_grads([("dQ", got[0], ref[0]), ("dK", got[1], ref[1]), ("dV", got[2], ref[2])], tag="outlier channel bwd")


def _rising_scores(B, Hq, Hkv, S, D, seed, rise_log2=150.0):
    """N(0,1) inputs with channel 0 of Q set to 16 and channel 0 of K rising linearly along the sequence, so
    that a row's scores grow by up to `rise_log2` (log2 units) between its first and its last keys."""
    x = si.make_inputs(B, Hq, Hkv, S, D, seed, with_do=True)
    c = 1.0 / np.sqrt(D) * np.log2(np.e)
    q = si.bf16_bits_to_f64(x.q_bits)
    k = si.bf16_bits_to_f64(x.k_bits)
    q[..., 0] = 16.0
    k[..., 0] = np.arange(S)[None, :, None] * (rise_log2 / (16.0 * c * S))
    x.q_bits = si.bf16_bits_from_f32(q.astype(np.float32))
    x.k_bits = si.bf16_bits_from_f32(k.astype(np.float32))
    return x


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [(1, 4, 2, 1536, 128, True), (1, 2, 1, 1200, 64, False)])
def test_rising_scores_redo_with_the_tracked_maximum(B, Hq, Hkv, S, D, causal, monkeypatch):
    """Scores rising by up to 150 (log2 units) along each row: for the later rows a tile's probabilities
    overflow the first tile's maximum (a lane's tile sum passes 2^64), so those waves redo their rows with the
    tracked maximum while the earlier ones keep the first pass. Both block geometries meet the oracle bar
    (O within the bound of the kernel's rounding, as for the other peaky inputs) and agree bitwise. The gradients are compared
    with the oracle's gradients given the kernel's O at a doubled stress budget, rel-L2 <= 2e-2: with one
    dominant key per row and neighbouring keys alike in the rising channel, a dQ row is a small difference
    of terms whose bf16 rounding (dS for the dQ MFMA) does not cancel (1.1e-2 measured for the non-causal
    rows, where every row is peaky)."""
    import torch
    lca = _lib()
    print(f"case rising scores B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal}", flush=True)
    x = _rising_scores(B, Hq, Hkv, S, D, 57)
    outs = []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        o, got, ref, _ = _run_bits(B, Hq, Hkv, S, D, causal, x, f"rising scores waves={waves}", stress=True)
        errs = [rel_l2(g, r) for g, r in zip(got, ref)]
        print(f"rising scores waves={waves} bwd: dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
        assert all(np.all(np.isfinite(g)) for g in got) and max(errs) <= 2 * TOL_GRAD_REL
        outs.append(o)
    assert np.array_equal(outs[0], outs[1])
    # the ring-merge forward redoes the same waves: into an empty running result it gives the forward's O, LSE
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    scale = 1.0 / np.sqrt(D)
    o_acc = torch.empty((B, S, Hq, D), dtype=torch.float32, device="cuda")
    l_acc = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o_out = torch.empty_like(q)
    lca.fwd_merge(q, k, v, o_acc, l_acc, causal=causal, accumulate=False, o_out=o_out, scale=scale)
    torch.cuda.synchronize()
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=causal, scale=scale, workers=None)
    check_fwd(host(o_out), host(l_acc), ro, rl, tag="rising scores fwd_merge",
              bound=_stress_bound(host(o_out), ro, qv, kv, vv, causal, scale))


def test_rising_scores_with_a_key_split():
    """The same inputs on a grid small enough for the forward's key split: each share keeps its own first-tile
    maximum or redoes, and the combine meets the oracle bar."""
    import torch
    lca = _lib()
    B, Hq, Hkv, S, D = 1, 1, 1, 8192, 128
    print(f"case rising scores, key split B={B} Hq={Hq} S={S}", flush=True)
    x = _rising_scores(B, Hq, Hkv, S, D, 59)
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    scale = 1.0 / np.sqrt(D)
    qv, kv, vv = x.values("q"), x.values("k"), x.values("v")
    ro, rl = oracle.attention_fwd(qv, kv, vv, causal=True, scale=scale, workers=None)
    for split in (True, False):
        o, lse = lca.fwd(q, k, v, causal=True, scale=scale, split=split)
        torch.cuda.synchronize()
        check_fwd(host(o), host(lse), ro, rl, tag=f"rising scores split={split}",
                  bound=_stress_bound(host(o), ro, qv, kv, vv, True, scale))


SPLIT = [
    # B, Hq, Hkv, S, D, causal, lengths, expected key split
    (1, 2, 1, 4096, 128, True, None, 2),
    (1, 1, 1, 8192, 64, False, None, 4),
    (1, 2, 1, 8192, 128, True, [3000, 5192], 4),
    (2, 1, 1, 5000, 64, True, None, 2),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths,ks", SPLIT)
def test_forward_key_split_matches_oracle(B, Hq, Hkv, S, D, causal, lengths, ks):
    """Small grids split each query block's key tiles over ks workgroups and combine the shares;
    the split and the unsplit forward both meet the oracle bar."""
    import torch
    lca = _lib()
    nbytes = lca.fwd_workspace_bytes(B, Hq, Hkv, S, D)
    assert nbytes == -(-4 * ks * B * S * Hq * D // 256) * 256 + 4 * ks * B * Hq * S
    print(f"case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} ks={ks}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 48, lengths=lengths, with_do=False)
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    ro, rl = oracle.attention_fwd(x.values("q"), x.values("k"), x.values("v"), causal=causal, scale=scale,
                                  cu_seqlens=x.cu_seqlens, workers=None)
    for split in (True, False):
        o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale, split=split)
        torch.cuda.synchronize()
        check_fwd(host(o), host(lse), ro, rl, tag=f"fwd split={split}")


def test_outputs_are_bitwise_deterministic():
    """No atomics: two runs on the same inputs give identical bits, with and without the split passes
    (the last case splits the forward's key tiles and the backward's heads and key tiles)."""
    import torch
    lca = _lib()
    for (B, Hq, Hkv, S, D, causal) in [(1, 8, 1, 1000, 128, True), (1, 28, 4, 8192, 128, True),
                                       (1, 2, 1, 8192, 128, True)]:
        print(f"case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal}", flush=True)
        x = si.make_inputs(B, Hq, Hkv, S, D, 47, with_do=True)
        q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
        runs = []
        for _ in range(2):
            o, lse = lca.fwd(q, k, v, causal=causal)
            dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=causal)
            torch.cuda.synchronize()
            runs.append([t.clone() for t in (o, lse, dq, dk, dv)])
        for a, b in zip(*runs):
            assert torch.equal(a, b)


GEOMETRY = [
    # B, Hq, Hkv, S, D, causal, lengths: 128-query (4 waves) and 256-query (8 waves) forward blocks
    (1, 4, 2, 1000, 128, True, None),
    (2, 3, 1, 700, 64, False, None),
    (1, 7, 1, 1000, 128, True, [100, 1, 1, 64, 65, 500, 269]),
    (1, 2, 2, 5000, 64, True, None),
    (1, 2, 1, 4500, 128, False, [4000, 500]),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths", GEOMETRY)
def test_forward_block_geometries_match_oracle_and_each_other(B, Hq, Hkv, S, D, causal, lengths, monkeypatch):
    """Both forward block geometries (ATTN_FWD_WAVES=4: 128-query blocks, 8: 256-query blocks sharing each
    K/V tile) meet the oracle bar and give bitwise the same O and LSE: every row is computed in the same order."""
    import torch
    lca = _lib()
    print(f"case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths}", flush=True)
    x = si.make_inputs(B, Hq, Hkv, S, D, 49, lengths=lengths, with_do=False)
    q, k, v = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits)
    cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
    scale = 1.0 / np.sqrt(D)
    ro, rl = oracle.attention_fwd(x.values("q"), x.values("k"), x.values("v"), causal=causal, scale=scale,
                                  cu_seqlens=x.cu_seqlens, workers=None)
    outs = []
    for waves in ("4", "8"):
        monkeypatch.setenv("ATTN_FWD_WAVES", waves)
        o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale, split=False)
        torch.cuda.synchronize()
        check_fwd(host(o), host(lse), ro, rl, tag=f"fwd waves={waves}")
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


FEW_KEYS = [
    # B, Hq, Hkv, S, D, causal, lengths, qk_std: sequences or segments under 64 keys, where the backward
    # takes Delta from its definition
    (1, 2, 1, 2, 64, True, None, 1.0),
    (2, 4, 2, 4, 128, True, None, 1.0),
    (1, 4, 2, 8, 64, True, None, 2.0),
    (1, 4, 2, 16, 128, False, None, 2.0),
    (2, 4, 1, 40, 64, True, None, 3.0),
    (1, 4, 2, 63, 128, False, None, 3.0),
    (1, 4, 2, 64, 128, True, [1, 2, 3, 5, 8, 13, 32], 1.0),
    (1, 6, 2, 64, 64, False, [2, 3, 4, 55], 2.0),
    (1, 4, 2, 200, 128, True, [2, 60, 64, 74], 2.0),  # rows on both sides of the 63-row boundary
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal,lengths,qk_std", FEW_KEYS)
def test_few_key_rows_backward_against_the_exact_gradient(B, Hq, Hkv, S, D, causal, lengths, qk_std):
    """Rows that see fewer than 64 keys, where softmax mass sits on a few keys so that dP_ij - Delta_i is a
    small difference: with Delta = dO . O from the bf16 O the rounding of O alone moves the gradients by up
    to 8e-3 rel-L2 on these shapes (fp64 computation from the oracle's gradients, 6 seeds each). The
    backward takes Delta_i = sum_j P_ij dP_ij there, so what is left is the bf16 rounding of P, dS and the
    outputs: the gradients of the forward's own O and LSE are held to rel-L2 <= 5e-3 of the exact ones,
    half the general bar, on three seeds."""
    import torch
    lca = _lib()
    for seed in (81, 82, 83):
        tag = f"few keys B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} lengths={lengths} " \
              f"qk_std={qk_std} seed={seed}"
        print(tag, flush=True)
        x = si.make_inputs(B, Hq, Hkv, S, D, seed, lengths=lengths, with_do=True, qk_std=qk_std)
        q, k, v, do = dev_bf16(x.q_bits), dev_bf16(x.k_bits), dev_bf16(x.v_bits), dev_bf16(x.do_bits)
        cu = dev_i32(x.cu_seqlens) if x.cu_seqlens is not None else None
        scale = 1.0 / np.sqrt(D)
        o, lse = lca.fwd(q, k, v, causal=causal, cu_seqlens=cu, scale=scale)
        dq, dk, dv = lca.bwd(q, k, v, o, lse, do, causal=causal, cu_seqlens=cu, scale=scale)
        torch.cuda.synchronize()
        qv, kv, vv, dov = (x.values(n) for n in ("q", "k", "v", "do"))
        rq, rk, rv = oracle.attention_bwd(qv, kv, vv, dov, causal=causal, scale=scale, cu_seqlens=x.cu_seqlens,
                                          workers=None)
        errs = [rel_l2(host(g), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
        print(f"{tag}: dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
        assert max(errs) <= 5e-3, tag
