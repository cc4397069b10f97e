// bf16 forward kernel for gfx950.
//
// The method is the tiled, fused attention of "ms-swift集成FlashAttention 2/3，
// 长文本训练更高效" (section "FlashAttention 如何破局"): a Q block stays on chip,
// K/V blocks stream through on-chip memory, and a running maximum plus
// normaliser per row replace the full softmax, so only O (and the
// log-sum-exp) reach global memory. The FA-2 paragraph of the same page names
// double-buffered loads; here K and V tiles are double-buffered through LDS.
//
// Work split: one workgroup of 4 waves per (b, h_q, 128 queries), two
// workgroups per CU (two waves per SIMD, so one wave's softmax overlaps the
// other's MFMAs; at most 256 VGPRs each); or, for long unpacked sequences,
// 8 waves per (b, h_q, 256 queries), one workgroup per CU sharing each K/V
// tile (fwd_block_waves()).
//   * Each wave owns 32 queries. Its Q slice sits in VGPRs as the B operand of
//     S^T = K Q^T, so every lane owns one query column and the row statistics
//     need only one exchange between the two lane halves (v_permlane32_swap).
//   * K rows are read through perm_rows, which leaves the probabilities in
//     exactly the register order the B operand of O^T += V^T P^T needs.
//   * V^T fragments come from the transposing LDS read; V stays row-major.
//   * K/V tiles (64 keys) move from global memory straight into LDS
//     (buffer_load_dwordx4 ... lds, no staging registers), double-buffered
//     with one barrier per tile.
//   * Software pipeline: the scores of tile j + 1 are computed in the same
//     straight block as the exp/sum/pack of tile j, so their MFMAs interleave
//     with the softmax VALU work; K is kept one tile ahead of V.
//   * Running maximum: a row's maximum over the first tile where it sees
//     keys, kept for the rest of the row. The online softmax only needs some
//     common offset per row that keeps the probabilities in range; for the
//     scores met in practice the first tile's maximum does, so the later
//     tiles compute no maximum and never rescale (5-7 % of the kernel's time
//     on MI355X against tracking the maximum with a lazy rescale). A wave in
//     which a lane's probability sum over a tile passes 2^64 (scores rising
//     by ~64 in log2 units past the row's first tile) redoes its rows with
//     the tracked maximum.
//   * Tiles partly (or wholly) outside a wave's visible keys are masked per
//     element. Every LDS address is a per-lane base computed once plus a
//     compile-time offset, and every per-tile branch is scalar.
//   * Rows that see fewer than 64 keys are recomputed afterwards in fp32 by
//     attn_fwd_fewkeys_kernel.
//   * Key split (grids too small to fill the GPU, chosen on the host): the key
//     tiles of a query block are shared over key_split workgroups, which write
//     fp32 partial results; attn_fwd_combine_kernel merges them.
//   * Ring merge (attn_fwd_merge): the same kernels, with epilogues that fold
//     the call's result into a running fp32 (O, LSE) (the Ring-Attention
//     paragraph of the page's sequence-parallel section accumulates partial
//     results per arriving K/V block) instead of writing O and LSE.
#define ATTN_LDS_FAULT_WORD g_lds_fault_fwd
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

constexpr int kBN = 64;  // keys per tile
// Rows that see fewer keys than this are recomputed (or, in a ring merge,
// merged) by attn_fwd_fewkeys_kernel, not by the tiled kernel.
constexpr int kFewKeys = kFewKeyLimit;

// WAVES waves of 32 queries per workgroup: 4 (128-query blocks, two
// workgroups per CU) or 8 (256-query blocks, one workgroup per CU, so each
// K/V tile is copied into LDS once per CU); fwd_block_waves() picks one.
// With D = 64 the kernel is held to 128 VGPRs so that four waves run per SIMD
// (it spills 20 bytes per lane; 1-4 % faster than three waves at 161 VGPRs).
// MERGE: the epilogue folds the result into the running (o_acc, lse_acc)
// of a ring step instead of writing o and lse.
template <int D, bool CAUSAL, int WAVES, bool MERGE>
__global__ __launch_bounds__(WAVES * 64, (D == 64 ? 16 : 8) / WAVES) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int kWaves = WAVES;
  constexpr int kBM = 32 * kWaves;
  constexpr int KS = D / 16;     // k-steps of the score product
  constexpr int DB = D / 32;     // 32-wide d blocks of the output
  constexpr int TILE = kBN * D;  // elements of one K or V tile
  constexpr int NI = TILE * 2 / (kWaves * 1024);  // DMA instructions per wave per tensor and tile
  // The two buffers are separate objects so that alias analysis can tell the
  // reads of one from the DMA writes into the other (no waits between them).
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[TILE];
  __shared__ int red[2][kWaves];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int hq = bh - b * p.hq;
  const int hk = hq / (p.hq / p.hkv);
  // blockIdx.y = rank * key_split + share, ranks from the heaviest block
  // (the last one) down; with a key split the shares of a block run together
  const int ks = p.key_split;
  const int yrank = (int)blockIdx.y / ks;
  const int share = (int)blockIdx.y - yrank * ks;
  const int qblk = p.num_qblk - 1 - yrank;
  const int my_q = qblk * kBM + wave * 32 + n;
  const bool q_ok = my_q < p.seqlen;

  const int q_stride = p.hq * D;
  const int kv_stride = p.hkv * D;
  const __bf16* qg = p.q + (size_t)b * p.seqlen * q_stride + hq * D;
  const __bf16* kg = p.k + (size_t)b * p.seqlen * kv_stride + hk * D;
  const __bf16* vg = p.v + (size_t)b * p.seqlen * kv_stride + hk * D;

  // visible keys of this lane's query: [kstart, kend)
  int kstart = 0, kend = 0;
  if (q_ok) {
    int s0, s1;
    segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, my_q, s0, s1);
    kstart = s0;
    kend = CAUSAL ? my_q + 1 : s1;
  }
  // Wave bounds: a tile is skipped when it misses every visible range of the
  // wave and unmasked when it lies inside all of them. The reductions are
  // wave-uniform; readfirstlane says so, which keeps the tile branches scalar.
  const int lo_min = __builtin_amdgcn_readfirstlane(wave_min(q_ok ? kstart : INT32_MAX));
  const int hi_max = __builtin_amdgcn_readfirstlane(wave_max(q_ok ? kend : INT32_MIN));
  const int lo_max = __builtin_amdgcn_readfirstlane(wave_max(q_ok ? kstart : INT32_MIN));
  const int hi_min = __builtin_amdgcn_readfirstlane(wave_min(q_ok ? kend : INT32_MAX));
  if (lane == 0) {
    red[0][wave] = lo_min;
    red[1][wave] = hi_max;
  }
  __syncthreads();
  int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wg_lo = min(wg_lo, red[0][w]);
    wg_hi = max(wg_hi, red[1][w]);
  }
  wg_lo = __builtin_amdgcn_readfirstlane(wg_lo);
  wg_hi = __builtin_amdgcn_readfirstlane(wg_hi);
  const int blk_begin = wg_hi > wg_lo ? wg_lo / kBN : 0;
  const int blk_tiles = wg_hi > wg_lo ? (wg_hi + kBN - 1) / kBN - blk_begin : 0;
  // this workgroup's share of the block's key tiles (all of them without a split)
  const int tile_begin = blk_begin + share * blk_tiles / ks;
  const int tile_end = blk_begin + (share + 1) * blk_tiles / ks;

  // Q slice as B operands: lane (n, h) holds Q[my_q][16t + 8h .. +7]
  bf16x8 qf[KS];
  {
    const __bf16* qrow = qg + (size_t)min(my_q, p.seqlen - 1) * q_stride + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[t] = as_bf16x8(load16(qrow + 16 * t));
  }

  // Per-lane LDS element offsets (tile-relative).
  int koff[KS];  // K row perm_rows(n), chunk 2t + h: A operand of S^T, key block 0
#pragma unroll
  for (int t = 0; t < KS; ++t) koff[t] = row_frag_b128<D>(lane, t);
  int voff[DB];  // first transposing read of the V^T fragment (key step 0, d block db)
#pragma unroll
  for (int db = 0; db < DB; ++db) voff[db] = tr_frag_tr<D>(lane, db, 0);

  // DMA tile loader. Instruction i of wave w fills the 1 KiB of LDS at
  // (4 i + w) KiB of the tile, lane L the 16 bytes at L * 16 of it: tile row
  // `row`, physical chunk `pc`. The lane fetches the logical chunk that the
  // swizzle puts there (both swizzles are XORs, hence involutions). The
  // buffer resource starts at the tile's first row and ends at the last key,
  // so rows past the end read as zeros (their keys are masked anyway).
  uint32_t ld_koff[NI], ld_voff[NI];  // byte offsets within the tile
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = tile_dma_elem(i, kWaves, wave, lane);  // element offset in the tile
    ld_koff[i] = dma_src_b128<D>(e, kv_stride);
    ld_voff[i] = dma_src_tr<D>(e, kv_stride);
  }
  auto issue_k = [&](int t0, auto buf_c) {
    __bf16* kd = decltype(buf_c)::value ? k_lds1 : k_lds0;
    const uint32_t nbytes = (uint32_t)(p.seqlen - t0) * (uint32_t)kv_stride * 2u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)t0 * kv_stride, nbytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_buf(rk, ld_koff[i], kd + tile_dma_elem(i, kWaves, wave, 0));
  };
  auto issue_v = [&](int t0, auto buf_c) {
    __bf16* vd = decltype(buf_c)::value ? v_lds1 : v_lds0;
    const uint32_t nbytes = (uint32_t)(p.seqlen - t0) * (uint32_t)kv_stride * 2u;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)t0 * kv_stride, nbytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_buf(rv, ld_voff[i], vd + tile_dma_elem(i, kWaves, wave, 0));
  };
  // S^T of one tile: the two 32-key chains alternate, and the K operands of
  // step t + 2 are read before the MFMAs of step t, so the LDS latency
  // overlaps MFMAs instead of stalling each one.
  auto scores = [&](const __bf16* ks, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
    bf16x8 a[3][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) a[t][kb] = lds_read_b128(ks, koff[t] + kb * 32 * D);
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t + 2 < KS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) a[(t + 2) % 3][kb] = lds_read_b128(ks, koff[t + 2] + kb * 32 * D);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(a[t % 3][kb], qf[t], s[kb]);
    }
  };

  f32x16 acc[DB];
  float m_run;  // running maximum (scaled, log2 units)
  float l_run;  // partial row sum over this lane's keys
  const float c = p.scale_log2e;
  const int ntile = tile_end - tile_begin;

  // First key tile of this lane's row within this workgroup's share.
  const int kfirst = max(kstart, tile_begin * kBN) / kBN * kBN;

  // One pass over the workgroup's tiles. FAST: the running maximum of a row
  // is its maximum over the first tile where it sees keys, and it stays
  // there: no tile maximum and no rescale afterwards. That is exact as long
  // as no probability overflows; the pass returns whether some lane's sum
  // over a tile went above 2^64 (it cannot underflow: the first tile's
  // largest probability is 1). !FAST: the maximum follows every tile with
  // the lazy rescale. A wave that is not `active` only copies tiles and
  // meets the barriers, keeping its results.
  //
  // Software pipeline: the scores of tile j + 1 are computed while the
  // softmax of tile j runs, so K is kept one tile ahead of V. Tile
  // tile_begin + i has its K in buffer i & 1 and its V in buffer i & 1.
  auto run_tiles = [&](auto fast_c, bool active) {
    constexpr bool FAST = decltype(fast_c)::value;
    if (active) {
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
      m_run = kMaxInit;
      l_run = 0.f;
    }
    bool over = false;
    f32x16 s_cur[2];
    if (ntile > 0) {
      issue_k(tile_begin * kBN, std::integral_constant<int, 0>{});
      issue_v(tile_begin * kBN, std::integral_constant<int, 0>{});
      if (ntile > 1) issue_k((tile_begin + 1) * kBN, std::integral_constant<int, 1>{});
    }
    wait_dma();
    __syncthreads();
    if (active && ntile > 0) scores(k_lds0, s_cur);
    __syncthreads();  // K of the first tile is read before its buffer is refilled

    auto body = [&](int i, auto par_c) {
      constexpr int par = decltype(par_c)::value;
      const int t0 = (tile_begin + i) * kBN;
      if (i + 2 < ntile) issue_k(t0 + 2 * kBN, std::integral_constant<int, par>{});
      if (i + 1 < ntile) issue_v(t0 + kBN, std::integral_constant<int, par ^ 1>{});
      if (active) {
        // Tiles a wave cannot see at all are fully masked (no per-wave
        // skipping, which keeps the loop body one straight block).
        const bool full = (t0 >= lo_max) && (t0 + kBN <= hi_min);
        if (!full) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t0 + kb * 32 + c_key(r, h);
              s_cur[kb][r] = (key < kstart || key >= kend) ? -INFINITY : s_cur[kb][r];
            }
        }
        if (!FAST || __any(t0 == kfirst)) {
          float mx = fmaxf(s_cur[0][0], s_cur[1][0]);
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = max3f(mx, s_cur[0][r], s_cur[1][r]);
          const float m_tile = max_lane_halves(mx) * c;
          if (FAST) {
            // rows entering their first tile (a row without keys here keeps
            // kMaxInit, and all its probabilities are 0)
            if (t0 == kfirst && m_tile > kMaxInit) m_run = m_tile;
          } else if (__any(m_tile > m_run + kRescaleThreshold)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int k = 0; k < DB; ++k) acc[k] *= alpha;
            m_run = m_new;
          }
        }
        // scores of the next tile (its K is already in LDS); on the last tile
        // this reads a stale buffer and the result is dropped
        f32x16 s_nxt[2];
        scores(par ? k_lds0 : k_lds1, s_nxt);
        const float neg_m = -m_run;
        bf16x8 pb[4];
        float lp[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: no serial chain of adds
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float e[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            e[r] = fast_exp2(__builtin_fmaf(s_cur[kb][r], c, neg_m));
            lp[r & 3] += e[r];
          }
          pb[2 * kb] = pack_bf16(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
          pb[2 * kb + 1] = pack_bf16(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
        }
        const float l_tile = (lp[0] + lp[1]) + (lp[2] + lp[3]);
        if (FAST) over = over || !(l_tile <= kTileSumLimit);
        l_run += l_tile;
        const __bf16* vs = par ? v_lds1 : v_lds0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32(tr_read_pair(vs, voff[db] + 16 * u * D, 4 * D), pb[u], acc[db]);
        s_cur[0] = s_nxt[0];
        s_cur[1] = s_nxt[1];
      }
      wait_dma();
      __syncthreads();
    };

    for (int i = 0; i < ntile; i += 2) {
      body(i, std::integral_constant<int, 0>{});
      if (i + 1 < ntile) body(i + 1, std::integral_constant<int, 1>{});
    }
    return over;
  };

  // The fast pass, then, for the waves where a probability overflowed, the
  // pass with the tracked maximum (rare: scores rising by more than 64 in
  // log2 units past a row's first tile). Redoing whole waves keeps every row's
  // result independent of the workgroup's other waves.
  const bool redo = __any(run_tiles(std::true_type{}, true));
  if (__syncthreads_or(redo)) run_tiles(std::false_type{}, redo);

  // epilogue: O = acc / l, LSE = (m + log2 l) * ln 2; with a key split the
  // share's fp32 O and m + log2 l, combined by attn_fwd_combine_kernel; in a
  // ring merge, the merge of (acc / l, m + log2 l) into the running result
  const float l_tot = sum_lane_halves(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok && ks > 1) {
    const size_t plane = (size_t)p.batch * p.seqlen * q_stride;
    float* orow = p.part_o + (size_t)share * plane + ((size_t)b * p.seqlen + my_q) * q_stride + hq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (h == 0) {
      p.part_lse[(((size_t)share * p.batch + b) * p.hq + hq) * p.seqlen + my_q] =
          l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
    }
  } else if (MERGE) {
    // A row that sees at least 64 keys has l > 0. With the running result's
    // L_a = LSE_acc log2 e and this call's L_p = m + log2 l, M = max(L_a, L_p),
    // w_a = 2^(L_a - M), w_p = 2^(L_p - M), T = w_a + w_p:
    //   O = (w_a O_acc + w_p acc / l) / T = (w_a / T) O_acc + (2^(m - M) / T) acc,
    //   LSE = (M + log2 T) ln 2.
    // The two lanes of a row both read LSE_acc before the h = 0 lane stores
    // the new one (the store depends on the loaded value).
    if (q_ok && kend - kstart >= kFewKeys) {
      const size_t ri = ((size_t)b * p.seqlen + my_q) * q_stride + hq * D;
      const size_t li = ((size_t)b * p.hq + hq) * p.seqlen + my_q;
      const float la = p.accumulate ? p.lse_acc[li] * kLog2e : -INFINITY;
      const float lp = m_run + __log2f(l_tot);
      const float mm = fmaxf(la, lp);
      const float wa = fast_exp2(la - mm);  // 0 for an empty running result
      const float tot = wa + fast_exp2(lp - mm);
      const float rt = 1.0f / tot;
      const float ca = wa * rt, cp = fast_exp2(m_run - mm) * rt;
      float* arow = p.o_acc + ri;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* dst = reinterpret_cast<f32x4*>(arow + 32 * db + 8 * g + 4 * h);
          const f32x4 old = p.accumulate ? *dst : f32x4{};
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = ca * old[e] + cp * acc[db][4 * g + e];
          *dst = w;
          if (p.o_out != nullptr) {
            bf16x4 wb;
#pragma unroll
            for (int e = 0; e < 4; ++e) wb[e] = (__bf16)w[e];
            *reinterpret_cast<bf16x4*>(p.o_out + ri + 32 * db + 8 * g + 4 * h) = wb;
          }
        }
      if (h == 0) p.lse_acc[li] = (mm + __log2f(tot)) * kLn2;
    }
  } else if (q_ok) {
    __bf16* orow = p.o + ((size_t)b * p.seqlen + my_q) * q_stride + hq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
        w[0] = (__bf16)(acc[db][4 * g + 0] * inv);
        w[1] = (__bf16)(acc[db][4 * g + 1] * inv);
        w[2] = (__bf16)(acc[db][4 * g + 2] * inv);
        w[3] = (__bf16)(acc[db][4 * g + 3] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (h == 0) {
      p.lse[((size_t)b * p.hq + hq) * p.seqlen + my_q] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Key-split combine: for each (b, s, h_q) row and shares s = 1..ks with
// partial outputs O_s and L_s = m_s + log2 l_s,
//   O = sum_s 2^(L_s - M) O_s / sum_s 2^(L_s - M),  M = max_s L_s,
//   LSE = (M + log2 sum_s 2^(L_s - M)) ln 2.
// One thread per 8 consecutive d of a row; the D / 8 threads of a row sit in
// one wave. HBM-bound: 4 ks bytes read and 2 written per output element.
// In a ring merge (o_acc set) the combined (O, L) is folded into the running
// result as the tiled kernel's merge epilogue does; for the bf16 forward
// (few_rows_apart) rows with fewer than 64 visible keys are left to
// attn_fwd_fewkeys_kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_combine_kernel(FwdParams p) {
  constexpr int T = D / 8;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rows = (size_t)p.batch * p.seqlen * p.hq;
  const size_t row = gid / T;  // (b * S + s) * Hq + h
  const int sub = (int)(gid % T);
  if (row >= rows) return;
  const int hq = (int)(row % p.hq);
  const size_t bs = row / p.hq;
  const int s = (int)(bs % p.seqlen);
  const int b = (int)(bs / p.seqlen);
  const int ks = p.key_split;
  const size_t lstride = (size_t)p.batch * p.hq * p.seqlen;
  const size_t li = ((size_t)b * p.hq + hq) * p.seqlen + s;
  if (p.o_acc != nullptr && p.few_rows_apart) {
    int s0, s1;
    segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, s, s0, s1);
    if ((p.causal ? s + 1 : s1) - s0 < kFewKeys) return;  // whole rows, so no lane waits on another
  }
  float m = -INFINITY;
  for (int sp = 0; sp < ks; ++sp) m = fmaxf(m, p.part_lse[sp * lstride + li]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m > -INFINITY) {
    const size_t plane = rows * D;
    for (int sp = 0; sp < ks; ++sp) {
      const float w = fast_exp2(p.part_lse[sp * lstride + li] - m);  // 0 for a share without keys
      tot += w;
      const f32x4* src = reinterpret_cast<const f32x4*>(p.part_o + sp * plane + row * D + 8 * sub);
      const f32x4 a = src[0], c = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * a[e];
        acc[4 + e] += w * c[e];
      }
    }
  }
  if (p.o_acc != nullptr) {
    // every share of a row that sees keys has l > 0, so tot > 0 for such a
    // row; acc / tot and m + log2 tot merged with the running result,
    // coefficients as in the tiled kernel
    const float la = p.accumulate ? p.lse_acc[li] * kLog2e : -INFINITY;
    const float lp = m + __log2f(tot);
    const float mm = fmaxf(la, lp);
    const float wa = fast_exp2(la - mm);
    const float t2 = wa + fast_exp2(lp - mm);
    const float rt = 1.0f / t2;
    const float ca = wa * rt, cp = fast_exp2(m - mm) * rt;
    f32x4* dst = reinterpret_cast<f32x4*>(p.o_acc + row * D + 8 * sub);
    const f32x4 a0 = p.accumulate ? dst[0] : f32x4{}, a1 = p.accumulate ? dst[1] : f32x4{};
    f32x4 r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = ca * a0[e] + cp * acc[e];
      r1[e] = ca * a1[e] + cp * acc[4 + e];
    }
    dst[0] = r0;
    dst[1] = r1;
    if (p.o_out != nullptr) {
      bf16x8 ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ob[e] = (__bf16)r0[e];
        ob[4 + e] = (__bf16)r1[e];
      }
      *reinterpret_cast<bf16x8*>(p.o_out + row * D + 8 * sub) = ob;
    }
    if (sub == 0) p.lse_acc[li] = (mm + __log2f(t2)) * kLn2;
    return;
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(p.o + row * D + 8 * sub) = out;
  if (sub == 0) p.lse[li] = tot > 0.f ? (m + __log2f(tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Rows that see fewer than 64 keys (the first 63 rows of every causal segment,
// and every row of a non-causal segment shorter than 64) carry their whole
// softmax on a handful of probabilities, so the bf16 rounding of P in the
// tiled kernel (up to 2^-8 relative) shows in their O. This kernel recomputes those
// rows exactly as the definition reads, in fp32 with unrounded
// probabilities, and overwrites their O and LSE: scores s_j = scale q . k_j,
// an online maximum and normaliser over the row's keys, O = sum_j p_j v_j / l,
// LSE = m + ln l.
// Workgroup (4-row block of a segment, h_q, b): the segment's first keys (at
// most 63) go to LDS, then one wave per row: lane j computes the score of key
// j, the wave takes the exact maximum and sum, and lane t accumulates
// O[d] = sum_j p_j v_j[d] for d = t, t + 64.
// In a ring merge (o_acc set) the exact (O, LSE) of the row is merged into the
// running result instead (the tiled kernel and the combine leave these rows
// alone): M = max(LSE_acc, LSE), w = e^(LSE - M) for each, O = (w_acc O_acc +
// w O) / (w_acc + w), LSE = M + ln(w_acc + w).
// ---------------------------------------------------------------------------
constexpr int kFewRowsPerWg = 4;  // one wave per row
constexpr int kFewBlocks = (kFewKeys + kFewRowsPerWg - 1) / kFewRowsPerWg;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_fewkeys_kernel(FwdParams p) {
  constexpr int C = D / 8;  // 16-byte chunks per row
  // K rows with chunk c of row j stored at chunk (c + j) % C, so that 64 lanes
  // reading one chunk each of 64 different rows hit different banks
  __shared__ __attribute__((aligned(16))) __bf16 ks[kFewKeys - 1][D];
  __shared__ __attribute__((aligned(16))) __bf16 vs[kFewKeys - 1][D];
  __shared__ __attribute__((aligned(16))) float qs[kFewRowsPerWg][D];
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int seg = (int)blockIdx.x / kFewBlocks;
  const int rblk = (int)blockIdx.x % kFewBlocks;
  int s0 = 0, s1 = p.seqlen;
  if (p.cu_seqlens != nullptr) {
    // clamped to [0, seqlen): a malformed array gives meaningless rows, never a stray address
    s0 = max(0, min(p.cu_seqlens[seg], p.seqlen));
    s1 = max(s0, min(p.cu_seqlens[seg + 1], p.seqlen));
  }
  const int len = s1 - s0;
  // these rows see keys [s0, s0 + nrows) only
  const int nrows = few_key_rows(len, CAUSAL);
  if (rblk * kFewRowsPerWg >= nrows) return;  // uniform over the workgroup
  const int hk = hq / (p.hq / p.hkv);
  const size_t q_stride = (size_t)p.hq * D, kv_stride = (size_t)p.hkv * D;
  const __bf16* kg = p.k + ((size_t)b * p.seqlen + s0) * kv_stride + hk * D;
  const __bf16* vg = p.v + ((size_t)b * p.seqlen + s0) * kv_stride + hk * D;
  const int tid = threadIdx.x;
  for (int e = tid; e < nrows * C; e += 256) {
    const int j = e / C, c = e % C;
    lds_store16g(&ks[j][((c + j) % C) * 8], load16(kg + (size_t)j * kv_stride + c * 8));
    lds_store16g(&vs[j][c * 8], load16(vg + (size_t)j * kv_stride + c * 8));
  }
  for (int e = tid; e < kFewRowsPerWg * D; e += 256) {
    const int w = e / D, d = e % D;
    const int rl = min(rblk * kFewRowsPerWg + w, nrows - 1);
    qs[w][d] = (float)p.q[((size_t)b * p.seqlen + s0 + rl) * q_stride + hq * D + d];
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int row_local = rblk * kFewRowsPerWg + wave;
  if (row_local >= nrows) return;  // whole waves leave
  const int r = s0 + row_local;
  const int nk = CAUSAL ? row_local + 1 : nrows;  // keys s0 .. s0 + nk - 1
  float sc = -INFINITY;
  if (lane < nk) {
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bf16x8 kv = lds_load16<bf16x8>(&ks[lane][((c + lane) % C) * 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qs[wave][c * 8 + e], (float)kv[e], dot);
    }
    sc = dot * p.scale;
  }
  float m = sc;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
  const float pj = lane < nk ? expf(sc - m) : 0.f;
  float l = pj;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) l += __shfl_xor(l, x);
  constexpr int DL = D / 64;  // d per lane
  float o[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) o[i] = 0.f;
  for (int j = 0; j < nk; ++j) {
    const float pb = __shfl(pj, j);
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] = __builtin_fmaf(pb, (float)vs[j][lane + 64 * i], o[i]);
  }
  const size_t ri = ((size_t)b * p.seqlen + r) * q_stride + hq * D;
  const size_t li = ((size_t)b * p.hq + hq) * p.seqlen + r;
  if (p.o_acc != nullptr) {
    // o / l has LSE m + ln l; its weight over the total is e^(m - M) l / T, so
    // its term is e^(m - M) o / T. Lane 0 stores LSE after every lane has read it.
    const float la = p.accumulate ? p.lse_acc[li] : -INFINITY;
    const float lp = m + logf(l);
    const float mm = fmaxf(la, lp);
    const float wa = expf(la - mm);  // 0 for an empty running result
    const float tot = wa + expf(lp - mm);
    const float ca = wa / tot, cp = expf(m - mm) / tot;
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      float* dst = p.o_acc + ri + lane + 64 * i;
      const float res = ca * (p.accumulate ? *dst : 0.f) + cp * o[i];
      *dst = res;
      if (p.o_out != nullptr) p.o_out[ri + lane + 64 * i] = (__bf16)res;
    }
    if (lane == 0) p.lse_acc[li] = mm + logf(tot);
    return;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < DL; ++i) p.o[ri + lane + 64 * i] = (__bf16)(o[i] * inv);
  if (lane == 0) p.lse[li] = m + logf(l);
}

template <int D, bool CAUSAL, bool MERGE>
void launch_tiled(const FwdParams& q, int waves, dim3 grid, hipStream_t stream) {
  if (waves == 8) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, 8, MERGE>), grid, dim3(8 * 64), 0, stream, q);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, 4, MERGE>), grid, dim3(4 * 64), 0, stream, q);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  if (q.key_split < 1 || q.part_o == nullptr || q.part_lse == nullptr) q.key_split = 1;
  const int waves = q.key_split > 1 ? 4 : fwd_block_waves(q.seqlen, D, q.causal, q.cu_seqlens != nullptr);
  q.num_qblk = (p.seqlen + 32 * waves - 1) / (32 * waves);
  dim3 grid(p.batch * p.hq, q.num_qblk * q.key_split);
  // with a key split the tiled kernel writes only partials, which the combine merges
  if (q.o_acc != nullptr && q.key_split == 1) {
    launch_tiled<D, CAUSAL, true>(q, waves, grid, stream);
  } else {
    launch_tiled<D, CAUSAL, false>(q, waves, grid, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (q.key_split > 1) {
    e = run_fwd_combine(q, stream);
    if (e != hipSuccess) return e;
  }
  // rows with fewer than 64 visible keys: none for a dense non-causal call with S >= 64
  if (CAUSAL || q.cu_seqlens != nullptr || q.seqlen < kFewKeys) {
    const int nseg = q.cu_seqlens != nullptr ? q.num_seqs : 1;
    const dim3 fgrid((unsigned)nseg * kFewBlocks, q.hq, q.batch);
    hipLaunchKernelGGL((attn_fwd_fewkeys_kernel<D, CAUSAL>), fgrid, dim3(256), 0, stream, q);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t run_fwd_combine(const FwdParams& p, hipStream_t stream) {
  const size_t threads = (size_t)p.batch * p.seqlen * p.hq * (p.head_dim / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.head_dim == 128) {
    hipLaunchKernelGGL((attn_fwd_combine_kernel<128>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((attn_fwd_combine_kernel<64>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t run_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.head_dim == 128) {
    return p.causal ? launch_fwd<128, true>(p, stream) : launch_fwd<128, false>(p, stream);
  }
  return p.causal ? launch_fwd<64, true>(p, stream) : launch_fwd<64, false>(p, stream);
}

#ifdef ATTN_DEBUG
hipError_t lds_faults_fwd(unsigned int* out) { return take_lds_fault_word(out); }
#endif

}  // namespace mi355attn
