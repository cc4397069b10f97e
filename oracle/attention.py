"""fp64 reference attention: forward, backward and the FP8 E4M3 decoder.

Test infrastructure: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use this module. It shares no code with the GPU library.

What is computed (all in float64, every input upcast exactly):

* Attention is the score matrix QKᵀ scaled, a row softmax over the keys a
  query may see, and the product of those probabilities with V. The page
  "ms-swift集成FlashAttention 2/3，长文本训练更高效" defines it this way in its
  section on why standard attention is memory-hungry: three separate steps
  (QKᵀ, softmax, PV) over a [B, H, S, S] score tensor. The fused method in its
  "FlashAttention 如何破局" section reaches the same result without storing
  that tensor, and the page's FA-2/-3 section says the outputs stay
  numerically consistent. So this oracle is the unfused definition, not a
  tiled or online algorithm.
* The softmax subtracts the exact row maximum before exponentiating. That is
  the overflow guard the same "FlashAttention 如何破局" section names (a
  running maximum plus a normaliser). Here it is taken over the whole row in
  one pass, then the exponentials are summed in a second pass.
* LSE_i = M_i + ln(L_i) (natural log): the log of the softmax denominator of
  row i, with M_i the row maximum and L_i the sum of exp(s_ij - M_i).
* Masks. Causal: key j is visible to query i iff j <= i. Packed sequences (the
  packing of several samples into one long sequence in "ms-swift长文本训练秘诀：
  Ulysses并行技术解析" §5 and in the FlashAttention page's section on
  engineering results): additionally j must lie in the same segment as i,
  with segments given by int32 prefix sums ``cu_seqlens``. Non-causal packed
  means block-diagonal full attention.
* GQA: query head h uses key/value head h // (Hq / Hkv). The pages say nothing
  about grouping; this is the contiguous reading.
* Backward: the gradient of L = <O, dO> with respect to Q, K and V, written
  per query row from the definition. With P the row's probabilities:
  dV_j = sum_i P_ij dO_i; dP_ij = dO_i . V_j; Delta_i = dO_i . O_i;
  dS_ij = P_ij (dP_ij - Delta_i); dQ_i = scale sum_j dS_ij K_j;
  dK_j = scale sum_i dS_ij Q_i. For GQA, dK and dV sum over the query heads
  of a group. The FlashAttention page says the backward needs the
  intermediates again (its memory section), and the forward keeps only O and
  the log-sum-exp. Here P is simply recomputed from the scores.

* Merging: attention over two disjoint key sets combines into attention
  over their union (``merge_partials``), the step Ring-Attention repeats as
  K/V blocks travel around the ring.

Layout: Q, O, dO, dQ are [B, S, Hq, D]; K, V, dK, dV are [B, S, Hkv, D];
LSE is [B, Hq, S].
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Iterable, Optional, Sequence

import numpy as np

try:  # limit BLAS to one thread per worker so workers do not oversubscribe
    from threadpoolctl import threadpool_limits as _tp_limits
except Exception:  # pragma: no cover
    _tp_limits = None

ROW_BLOCK = 128


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------


def segment_bounds(seqlen: int, cu_seqlens: Optional[Sequence[int]]) -> tuple[np.ndarray, np.ndarray]:
    """Per-token [start, end) of the packed segment holding it (whole sequence if unpacked)."""
    start = np.zeros(seqlen, dtype=np.int64)
    end = np.full(seqlen, seqlen, dtype=np.int64)
    if cu_seqlens is not None:
        cu = [int(c) for c in cu_seqlens]
        if cu[0] != 0 or cu[-1] != seqlen or any(b <= a for a, b in zip(cu, cu[1:])):
            raise ValueError("cu_seqlens must start at 0, increase strictly and end at seqlen")
        for a, b in zip(cu, cu[1:]):
            start[a:b] = a
            end[a:b] = b
    return start, end


def allowed_key_range(i: int, causal: bool, seg_start: np.ndarray, seg_end: np.ndarray) -> tuple[int, int]:
    """Half-open range [lo, hi) of the keys query i may attend to."""
    lo = int(seg_start[i])
    hi = i + 1 if causal else int(seg_end[i])
    return lo, hi


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------


def _block_probs(qb: np.ndarray, kk: np.ndarray, rows: np.ndarray, klo: int, lo: np.ndarray, hi: np.ndarray,
                 scale: float):
    """Scores, probabilities, row max and row sum for query rows ``rows`` against keys kk (offset klo)."""
    s = scale * (qb @ kk.T)  # [R, K]
    j = klo + np.arange(kk.shape[0])
    allowed = (j[None, :] >= lo[:, None]) & (j[None, :] < hi[:, None])
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # masked entries: exp(-inf) = 0
    l_sum = np.sum(e, axis=1)
    p = e / np.where(empty, 1.0, l_sum)[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l_sum)))
    return p, lse


def _group_size(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // hkv


def _kv_head(h: int, group: int) -> int:
    """Key/value head read by query head h: consecutive groups of ``group`` query heads share one."""
    return h // group


def _row_blocks(seqlen: int, block: Optional[int] = None):
    block = ROW_BLOCK if block is None else block
    return [(r0, min(seqlen, r0 + block)) for r0 in range(0, seqlen, block)]


def _workers(workers: Optional[int]) -> int:
    if workers is None:
        workers = int(os.environ.get("ORACLE_WORKERS", "0")) or min(16, len(os.sched_getaffinity(0)))
    return max(1, int(workers))


def _run_partitioned(fn, tasks: list, workers: int):
    """Run ``fn(chunk)`` on a static interleaved split of ``tasks``; results in chunk order."""
    workers = max(1, min(workers, len(tasks))) if tasks else 1
    chunks = [tasks[w::workers] for w in range(workers)]
    if workers == 1:
        return [fn(chunks[0])]
    ctx = _tp_limits(limits=1) if _tp_limits is not None else None
    try:
        if ctx is not None:
            ctx.__enter__()
        with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, chunks))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def attention_fwd(q, k, v, *, causal: bool, scale: float, cu_seqlens=None, workers: Optional[int] = 1):
    """Full forward: returns (O [B,S,Hq,D], LSE [B,Hq,S]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need batch == 1")
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, S), dtype=np.float64)
    tasks = [(b, h, r0, r1) for b in range(B) for h in range(Hq) for (r0, r1) in _row_blocks(S)]

    def run(chunk):
        for b, h, r0, r1 in chunk:
            rows = np.arange(r0, r1)
            lo = seg_start[rows]
            hi = rows + 1 if causal else seg_end[rows]
            klo, khi = int(lo.min()), int(hi.max())
            kv = _kv_head(h, G)
            p, l_ = _block_probs(q[b, r0:r1, h], k[b, klo:khi, kv], rows, klo, lo, hi, scale)
            o[b, r0:r1, h] = p @ v[b, klo:khi, kv]
            lse[b, h, r0:r1] = l_
        return None

    _run_partitioned(run, tasks, _workers(workers))
    return o, lse


def attention_fwd_rows(q, k, v, picks: Iterable[tuple[int, int, int]], *, causal: bool, scale: float,
                       cu_seqlens=None):
    """Forward for selected (b, h_q, i) rows only: returns (O rows [n, D], LSE [n])."""
    q = np.asarray(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    picks = list(picks)
    o = np.zeros((len(picks), D), dtype=np.float64)
    lse = np.zeros(len(picks), dtype=np.float64)
    for n, (b, h, i) in enumerate(picks):
        lo, hi = allowed_key_range(i, causal, seg_start, seg_end)
        kk = np.asarray(k[b, lo:hi, _kv_head(h, G)], dtype=np.float64)
        vv = np.asarray(v[b, lo:hi, _kv_head(h, G)], dtype=np.float64)
        s = scale * (kk @ np.asarray(q[b, i, h], dtype=np.float64))
        m = np.max(s)
        e = np.exp(s - m)
        l_sum = np.sum(e)
        o[n] = (e / l_sum) @ vv
        lse[n] = m + np.log(l_sum)
    return o, lse


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------


def _bwd_rows_block(qb, kk, vv, dob, rows, klo, lo, hi, scale):
    """Per-row gradient contributions of a block of query rows (all in float64)."""
    p, _ = _block_probs(qb, kk, rows, klo, lo, hi, scale)
    ob = p @ vv
    delta = np.sum(dob * ob, axis=1)
    dp = dob @ vv.T
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ kk)
    dk = scale * (ds.T @ qb)
    dv = p.T @ dob
    return dq, dk, dv


def attention_bwd(q, k, v, do, *, causal: bool, scale: float, cu_seqlens=None, workers: Optional[int] = 1):
    """Full backward: returns (dQ, dK, dV) in float64 (recomputes the forward)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    dq = np.zeros_like(q)
    tasks = [(b, h, r0, r1) for b in range(B) for h in range(Hq) for (r0, r1) in _row_blocks(S)]

    def run(chunk):
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for b, h, r0, r1 in chunk:
            rows = np.arange(r0, r1)
            lo = seg_start[rows]
            hi = rows + 1 if causal else seg_end[rows]
            klo, khi = int(lo.min()), int(hi.max())
            kv = _kv_head(h, G)
            g_q, g_k, g_v = _bwd_rows_block(q[b, r0:r1, h], k[b, klo:khi, kv], v[b, klo:khi, kv],
                                            do[b, r0:r1, h], rows, klo, lo, hi, scale)
            dq[b, r0:r1, h] = g_q
            dk[b, klo:khi, kv] += g_k
            dv[b, klo:khi, kv] += g_v
        return dk, dv

    parts = _run_partitioned(run, tasks, _workers(workers))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for pk, pv in parts:
        dk += pk
        dv += pv
    return dq, dk, dv


def attention_bwd_group(q, k, v, do, *, b: int, kv_head: int, causal: bool, scale: float, cu_seqlens=None,
                        workers: Optional[int] = None):
    """Backward of one batch entry and one kv head, i.e. all G query heads of the group.

    Returns (dQ [S, G, D] of the group's query heads, dK [S, D], dV [S, D]).
    Inputs may be float32/float64 arrays of the full tensors; only the
    group's slices are read.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    kk_all = np.asarray(k[b, :, kv_head], dtype=np.float64)
    vv_all = np.asarray(v[b, :, kv_head], dtype=np.float64)
    qg = np.asarray(q[b, :, kv_head * G:(kv_head + 1) * G], dtype=np.float64)
    dog = np.asarray(do[b, :, kv_head * G:(kv_head + 1) * G], dtype=np.float64)
    dq = np.zeros((S, G, D), dtype=np.float64)
    # heavy (late) row blocks first so the static split stays balanced
    tasks = [(g, r0, r1) for (r0, r1) in reversed(_row_blocks(S)) for g in range(G)]

    def run(chunk):
        dk = np.zeros((S, D), dtype=np.float64)
        dv = np.zeros((S, D), dtype=np.float64)
        for g, r0, r1 in chunk:
            rows = np.arange(r0, r1)
            lo = seg_start[rows]
            hi = rows + 1 if causal else seg_end[rows]
            klo, khi = int(lo.min()), int(hi.max())
            g_q, g_k, g_v = _bwd_rows_block(qg[r0:r1, g], kk_all[klo:khi], vv_all[klo:khi], dog[r0:r1, g],
                                            rows, klo, lo, hi, scale)
            dq[r0:r1, g] = g_q
            dk[klo:khi] += g_k
            dv[klo:khi] += g_v
        return dk, dv

    parts = _run_partitioned(run, tasks, _workers(workers))
    dk = np.zeros((S, D), dtype=np.float64)
    dv = np.zeros((S, D), dtype=np.float64)
    for pk, pv in parts:
        dk += pk
        dv += pv
    return dq, dk, dv


def attention_dq_rows(q, k, v, do, picks: Iterable[tuple[int, int, int]], *, causal: bool, scale: float,
                      cu_seqlens=None):
    """dQ for selected (b, h_q, i) rows: each row needs only its own probabilities and Delta_i."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    picks = list(picks)
    out = np.zeros((len(picks), D), dtype=np.float64)
    for n, (b, h, i) in enumerate(picks):
        lo, hi = allowed_key_range(i, causal, seg_start, seg_end)
        kk = np.asarray(k[b, lo:hi, _kv_head(h, G)], dtype=np.float64)
        vv = np.asarray(v[b, lo:hi, _kv_head(h, G)], dtype=np.float64)
        qi = np.asarray(q[b, i, h], dtype=np.float64)
        doi = np.asarray(do[b, i, h], dtype=np.float64)
        s = scale * (kk @ qi)
        e = np.exp(s - np.max(s))
        p = e / np.sum(e)
        oi = p @ vv
        delta = doi @ oi
        ds = p * (vv @ doi - delta)
        out[n] = scale * (ds @ kk)
    return out


def attention_dkdv_rows(q, k, v, do, picks: Iterable[tuple[int, int, int]], *, causal: bool, scale: float,
                        cu_seqlens=None, workers: Optional[int] = None):
    """dK and dV for selected (b, kv_head, j) key rows: returns (dK rows [n, D], dV rows [n, D]).

    Key j collects a term from every query row i that sees it, in each of the
    G query heads of its group: dV_j = sum_h sum_i P_ij dO_i and
    dK_j = scale sum_h sum_i P_ij (dO_i . V_j - Delta_i) Q_i, with
    P_ij = exp(s_ij - LSE_i) and Delta_i = dO_i . O_i. Those need LSE_i and O_i
    of every such row, so the group's full forward (attention_fwd on its query
    heads) runs first; the per-key sums then follow the definition directly.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _group_size(Hq, Hkv)
    seg_start, seg_end = segment_bounds(S, cu_seqlens)
    picks = list(picks)
    stats = {}
    for b, kvh in sorted({(int(b), int(kvh)) for b, kvh, _ in picks}):
        qg = np.asarray(q[b:b + 1, :, kvh * G:(kvh + 1) * G], dtype=np.float64)
        kg = np.asarray(k[b:b + 1, :, kvh:kvh + 1], dtype=np.float64)
        vg = np.asarray(v[b:b + 1, :, kvh:kvh + 1], dtype=np.float64)
        dog = np.asarray(do[b:b + 1, :, kvh * G:(kvh + 1) * G], dtype=np.float64)
        o, lse = attention_fwd(qg, kg, vg, causal=causal, scale=scale, cu_seqlens=cu_seqlens, workers=workers)
        delta = np.sum(dog[0] * o[0], axis=-1)  # [S, G]
        stats[(b, kvh)] = (qg[0], dog[0], lse[0], delta)
    dk = np.zeros((len(picks), D), dtype=np.float64)
    dv = np.zeros((len(picks), D), dtype=np.float64)
    for n, (b, kvh, j) in enumerate(picks):
        qg, dog, lse, delta = stats[(int(b), int(kvh))]
        # queries that see key j: same segment, and not before j when causal
        lo = j if causal else int(seg_start[j])
        hi = int(seg_end[j])
        kj = np.asarray(k[b, j, kvh], dtype=np.float64)
        vj = np.asarray(v[b, j, kvh], dtype=np.float64)
        for h in range(G):
            qi = qg[lo:hi, h]
            doi = dog[lo:hi, h]
            p = np.exp(scale * (qi @ kj) - lse[h, lo:hi])
            dv[n] += p @ doi
            ds = p * (doi @ vj - delta[lo:hi, h])
            dk[n] += scale * (ds @ qi)
    return dk, dv


# ---------------------------------------------------------------------------
# merging attention over disjoint key sets (Ring-Attention partials)
# ---------------------------------------------------------------------------


def merge_partials(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint key sets from the two parts.

    Ring-Attention passes K/V blocks around a ring and accumulates partial
    attention results locally until every device has seen the whole context
    (FlashAttention page, sequence-parallel section, Ring-Attention
    paragraph; "ms-swift支持GPU显存碎片整理提升利用率", section on
    Ring-Attention). The pages give no formula. From the definition: row i's
    softmax denominator over A ∪ B is e^{LSE_A} + e^{LSE_B}, and its output is
    the denominator-weighted mean of the two partial outputs:
        LSE = ln(e^{LSE_A} + e^{LSE_B}),
        O = (e^{LSE_A} O_A + e^{LSE_B} O_B) / e^{LSE}.
    Computed with the larger LSE factored out. A part with no visible key has
    LSE = -inf and weight 0; if both are empty, O = 0 and LSE = -inf.
    O [B, S, H, D], LSE [B, H, S]; returns (O, LSE) in float64.
    """
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    l1 = np.asarray(lse1, dtype=np.float64)
    l2 = np.asarray(lse2, dtype=np.float64)
    m = np.maximum(l1, l2)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - m_safe))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - m_safe))
    tot = w1 + w2
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    # weights are [B, H, S]; outputs [B, S, H, D]
    a1 = np.transpose(np.where(empty, 0.0, w1 / np.where(empty, 1.0, tot)), (0, 2, 1))[..., None]
    a2 = np.transpose(np.where(empty, 0.0, w2 / np.where(empty, 1.0, tot)), (0, 2, 1))[..., None]
    return a1 * o1 + a2 * o2, lse


# ---------------------------------------------------------------------------
# FP8 E4M3FN decoding (OCP 8-bit floating point, E4M3 variant)
# ---------------------------------------------------------------------------


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of OCP FP8 E4M3FN codes.

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the
    mantissa. Exponent 0 encodes subnormals m/8 * 2^-6. The all-ones pattern
    S.1111.111 is NaN. There is no infinity, so the largest finite magnitude
    is 1.75 * 2^8 = 448. FP8 appears on the FlashAttention page (FA-3 paragraph),
    and the E4M3 format with per-tensor scaling in the Q-Galore section of
    "ms-swift支持GPU显存碎片整理提升利用率".
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)
