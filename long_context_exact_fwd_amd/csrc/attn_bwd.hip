// bf16 backward kernels for gfx950: Delta, dK/dV, dQ.
//
// The backward recomputes the probabilities from the saved log-sum-exp
// instead of storing them. The FlashAttention page ("ms-swift集成FlashAttention
// 2/3，长文本训练更高效", section on why standard attention is memory-hungry)
// notes that the backward needs the intermediates again, and the fused
// forward keeps only O and the row statistics. With P_ij = exp(s_ij - LSE_i):
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . V_j
//   Delta_i = dO_i . O_i              dS_ij = P_ij (dP_ij - Delta_i)
//   dQ_i = scale sum_j dS_ij K_j      dK_j = scale sum_i dS_ij Q_i
// (Delta_i = sum_j P_ij dP_ij in rows that see fewer than 64 keys, where the
// bf16 rounding of the given O would dominate dP - Delta.)
// Split into two passes so that nothing is accumulated with atomics:
//   * dK/dV: one workgroup of 8 waves per (b, h_kv, 128 keys). Two waves share
//     each 32 keys: wave A holds K, computes S and P and accumulates dV^T;
//     wave B holds V, computes dP and, with A's P handed over through LDS,
//     dS and dK^T. Each wave then needs one accumulator and one operand set,
//     within 256 VGPRs, so two waves run per SIMD. B's dS and dK trail A's P
//     by one step, so within a step the two are independent, and their MFMA
//     and VALU phases alternate (one wave's exponentials or dS run under the
//     other's MFMAs). The loop covers every query head of the
//     GQA group and every visible 64-query tile, so the group sum needs no
//     reduction across workgroups.
//   * dQ: the forward's layout (waves of 32 queries; 4 per workgroup, two
//     workgroups per CU, or 8, one per CU, by the sizes): Q and dO stay in
//     VGPRs, K and V tiles stream through LDS.
// Tiles reach LDS through buffer loads that write LDS directly; rows past the
// sequence end read as zeros and are masked.
#define ATTN_LDS_FAULT_WORD g_lds_fault_bwd
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

constexpr int kQT = 64;  // queries per tile (dK/dV pass)
constexpr int kKT = 64;  // keys per tile (dQ pass)

// ---------------------------------------------------------------------------
// Work order. The dK/dV pass runs one workgroup per 128-row key block and
// share of the group's query heads, the dQ pass one per 128- or 256-row query
// block (dq_waves) and share of its key tiles, and a workgroup's
// cost is the number of 64-row tiles of the other operand it visits, times
// its heads. Under a causal or packed mask the costs differ by up to the
// longest segment over the tile size, and with a few workgroups per CU the
// launch order decides the makespan: both passes launch their work heaviest
// first (longest-processing-time order). For a single causal sequence this
// is key blocks from the start and query blocks from the end.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__device__ int block_tiles(const BwdParams& p, int pass, int blk) {
  const int rows = pass == 1 ? 32 * p.dq_waves : 128;
  const int r0 = blk * rows;
  const int r1 = min(r0 + rows, p.seqlen) - 1;
  int s0a, s1a, s0b, s1b;
  segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, r0, s0a, s1a);
  segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, r1, s0b, s1b);
  // pass 0: keys r0..r1 see queries [lo, hi); pass 1: queries r0..r1 see keys [lo, hi)
  const int lo = (pass == 0 && CAUSAL) ? r0 : s0a;
  const int hi = (pass == 1 && CAUSAL) ? r1 + 1 : s1b;
  return (hi + 63) / 64 - lo / 64;
}

// Entry e of a pass: dK/dV (pass 0) e = key block * head_split + share of the
// heads; dQ (pass 1) e = query block * key_split + share of the key tiles.
template <bool CAUSAL>
__device__ int entry_cost(const BwdParams& p, int pass, int e) {
  int lo, hi;
  if (pass == 1) {
    const int ns = p.key_split;
    share_range(block_tiles<CAUSAL>(p, 1, e / ns), ns, e % ns, lo, hi);
    return hi - lo;
  }
  const int ns = p.head_split;
  share_range(p.hq / p.hkv, ns, e % ns, lo, hi);
  return block_tiles<CAUSAL>(p, 0, e / ns) * (hi - lo);
}

// Rank of each entry by descending cost, ties by index; order[rank] = entry.
// Each thread ranks one entry against all of the pass, 256 at a time through LDS.
template <bool CAUSAL>
__device__ void block_order(const BwdParams& p, int wg) {
  __shared__ int cost[256];
  const int n0 = p.num_blk * p.head_split, n1 = p.num_dq_blk * p.key_split;
  const int c0 = (n0 + 255) / 256;
  const int pass = wg < c0 ? 0 : 1;
  const int n = pass == 0 ? n0 : n1;
  const int i = (pass == 0 ? wg : wg - c0) * 256 + (int)threadIdx.x;
  const int mine = i < n ? entry_cost<CAUSAL>(p, pass, i) : 0;
  int rank = 0;
  for (int c = 0; c < n; c += 256) {
    const int j = c + (int)threadIdx.x;
    __syncthreads();
    cost[threadIdx.x] = j < n ? entry_cost<CAUSAL>(p, pass, j) : INT32_MIN;
    __syncthreads();
    const int m = min(256, n - c);
    for (int t = 0; t < m; ++t) {
      const int cj = cost[t];
      rank += (cj > mine) || (cj == mine && c + t < i);
    }
  }
  if (i < n) p.order[(pass == 0 ? 0 : n0) + rank] = i;
}

// ---------------------------------------------------------------------------
// Delta_i = dO_i . O_i and LSE_i * log2(e), both fp32 [B, Hq, S] (the rows
// with fewer than 64 keys get their Delta again from the next kernel); the last
// ceil(num_blk * head_split / 256) + ceil(num_dq_blk * key_split / 256)
// workgroups write the work order instead.
// ---------------------------------------------------------------------------
// Rows per thread of the Delta kernel: all their loads are issued before the
// first product, so each thread keeps 2 * kDeltaRows 16-byte loads in flight.
constexpr int kDeltaRows = 4;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = D / 8;            // lanes per row, 16 bytes each
  constexpr int RPB = 256 / LPR;        // rows per pass of the workgroup
  constexpr int RPW = RPB * kDeltaRows;  // rows per workgroup
  // Rows are taken in the memory order of O and dO ([B, S, Hq, D]), so a wave
  // streams 64 / LPR consecutive rows. After them come the workgroups that
  // zero the padding rows [S, S64) of the statistics, then the work order.
  const long nrows = (long)p.batch * p.seqlen * p.hq;
  const int nstat = (int)((nrows + RPW - 1) / RPW);
  const int padw = p.stat_stride - p.seqlen;
  const long npad = (long)p.batch * p.hq * padw;
  const int npadwg = (int)((npad + 255) / 256);
  const int wg = (int)blockIdx.x;
  if (wg >= nstat + npadwg) {
    block_order<CAUSAL>(p, wg - nstat - npadwg);
    return;
  }
  if (wg >= nstat) {
    // padding rows get zeros: whole-tile copies read them and mask them
    const long j = (long)(wg - nstat) * 256 + threadIdx.x;
    if (j < npad) {
      const long r = (j / padw) * p.stat_stride + p.seqlen + (j % padw);
      p.delta[r] = 0.f;
      p.lse2[r] = 0.f;
    }
    return;
  }
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const long r0 = (long)wg * RPW + tid / LPR;
  // fp8 inputs: dP in the other kernels is dO . V8^T without descale_v, so
  // Delta is stored divided by it (V = 0 gives dS = 0 either way)
  float dv_inv = 1.f;
  if (p.descale_v != nullptr) {
    const float dv = p.descale_v[0];
    dv_inv = dv != 0.f ? 1.f / dv : 0.f;
  }
  bf16x8 av[kDeltaRows], gv[kDeltaRows];
#pragma unroll
  for (int k = 0; k < kDeltaRows; ++k) {
    const long r = min(r0 + (long)k * RPB, nrows - 1);  // rows past the end re-read the last one, unused
    av[k] = as_bf16x8(load16(p.o + r * D + sub * 8));
    gv[k] = as_bf16x8(load16(p.dout + r * D + sub * 8));
  }
#pragma unroll
  for (int k = 0; k < kDeltaRows; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)av[k][e] * (float)gv[k][e];
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    const long r = r0 + (long)k * RPB;  // (b * S + i) * Hq + h
    if (r < nrows && sub == 0) {
      const long hq = r % p.hq;
      const long bs = r / p.hq;
      const long i = bs % p.seqlen;
      const long bh = (bs / p.seqlen) * p.hq + hq;
      p.delta[bh * p.stat_stride + i] = dv_inv == 1.f ? acc : acc * dv_inv;
      p.lse2[bh * p.stat_stride + i] = p.lse[bh * p.seqlen + i] * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// Delta of the rows that see fewer than 64 keys, from its definition:
// Delta_i = sum_j P_ij dP_ij, with P_ij = exp2(s_ij c - LSE_i log2 e) and
// dP_ij = dO_i . V_j, instead of dO_i . O_i. O reaches the backward rounded
// to bf16; in a row whose softmax sits on a few keys, dP - Delta is a small
// difference that this rounding would dominate (a two-key row can lose the
// gradient's second digit). Launched after attn_bwd_delta_kernel in the
// Delta phase, over the first 63 rows of each causal segment (every row of
// a shorter non-causal segment), one wave per row and lane = key, as the
// forward's few-key kernel.
// The sum is Delta only if the call holds every key the row sees: a ring's
// chunk pair is called with the whole row's O and LSE, and keys of other
// chunks carry the rest of P. Given the row's LSE, sum_j P_ij over the call's
// keys is 1 exactly when no key is missing, so a row keeps dO . O unless that
// sum is within 2^-10 of 1 (then the missing keys hold at most that much of
// P, and change Delta by at most 2^-10 max |dP|, about the rounding of dO . O). With fp8 inputs q, k, v hold the E4M3 codes and c
// carries the descales of Q and K; dP then lacks d_v, which is how Delta is
// stored for those inputs.
// ---------------------------------------------------------------------------
constexpr int kFewRowsPerWgB = 4;  // one wave per row
constexpr float kWholeRowTol = 0.0009765625f;  // 2^-10
constexpr int kFewBlocksB = (kFewKeyLimit - 1 + kFewRowsPerWgB - 1) / kFewRowsPerWgB;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_delta_fewkeys_kernel(BwdParams p) {
  constexpr int C = D / 8;  // 16-byte chunks per row
  // K and V rows with chunk c of row j stored at chunk (c + j) % C, so that
  // 64 lanes reading one chunk each of 64 different rows hit different banks
  __shared__ __attribute__((aligned(16))) __bf16 ks[kFewKeyLimit - 1][D];
  __shared__ __attribute__((aligned(16))) __bf16 vs[kFewKeyLimit - 1][D];
  __shared__ __attribute__((aligned(16))) float qs[kFewRowsPerWgB][D];
  __shared__ __attribute__((aligned(16))) float gs[kFewRowsPerWgB][D];
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int seg = (int)blockIdx.x / kFewBlocksB;
  const int rblk = (int)blockIdx.x % kFewBlocksB;
  int s0 = 0, s1 = p.seqlen;
  if (p.cu_seqlens != nullptr) {
    // clamped to [0, seqlen): a malformed array gives meaningless rows, never a stray address
    s0 = max(0, min(p.cu_seqlens[seg], p.seqlen));
    s1 = max(s0, min(p.cu_seqlens[seg + 1], p.seqlen));
  }
  const int len = s1 - s0;
  // these rows see keys [s0, s0 + nrows) only
  const int nrows = few_key_rows(len, CAUSAL);
  if (rblk * kFewRowsPerWgB >= nrows) return;  // uniform over the workgroup
  const int hk = hq / (p.hq / p.hkv);
  const size_t q_stride = (size_t)p.hq * D, kv_stride = (size_t)p.hkv * D;
  const __bf16* kg = p.k + ((size_t)b * p.seqlen + s0) * kv_stride + hk * D;
  const __bf16* vg = p.v + ((size_t)b * p.seqlen + s0) * kv_stride + hk * D;
  const int tid = threadIdx.x;
  for (int e = tid; e < nrows * C; e += 256) {
    const int j = e / C, cc = e % C;
    lds_store16g(&ks[j][((cc + j) % C) * 8], load16(kg + (size_t)j * kv_stride + cc * 8));
    lds_store16g(&vs[j][((cc + j) % C) * 8], load16(vg + (size_t)j * kv_stride + cc * 8));
  }
  for (int e = tid; e < kFewRowsPerWgB * D; e += 256) {
    const int w = e / D, d = e % D;
    const int rl = min(rblk * kFewRowsPerWgB + w, nrows - 1);
    const size_t at = ((size_t)b * p.seqlen + s0 + rl) * q_stride + hq * D + d;
    qs[w][d] = (float)p.q[at];
    gs[w][d] = (float)p.dout[at];
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int row_local = rblk * kFewRowsPerWgB + wave;
  if (row_local >= nrows) return;  // whole waves leave
  const int r = s0 + row_local;
  const int nk = CAUSAL ? row_local + 1 : nrows;  // keys s0 .. s0 + nk - 1
  float c = p.scale_log2e;
  if (p.descale_q != nullptr) c = p.scale * p.descale_q[0] * p.descale_k[0] * kLog2e;
  const size_t bh = (size_t)b * p.hq + hq;
  const float lse2 = p.lse[bh * p.seqlen + r] * kLog2e;
  float pdp = 0.f, psum = 0.f;
  if (lane < nk) {
    float sdot = 0.f, gdot = 0.f;
#pragma unroll
    for (int cc = 0; cc < C; ++cc) {
      const bf16x8 kv = lds_load16<bf16x8>(&ks[lane][((cc + lane) % C) * 8]);
      const bf16x8 vv = lds_load16<bf16x8>(&vs[lane][((cc + lane) % C) * 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sdot = __builtin_fmaf(qs[wave][cc * 8 + e], (float)kv[e], sdot);
        gdot = __builtin_fmaf(gs[wave][cc * 8 + e], (float)vv[e], gdot);
      }
    }
    psum = exp2f(sdot * c - lse2);
    pdp = psum * gdot;
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    pdp += __shfl_xor(pdp, x);
    psum += __shfl_xor(psum, x);
  }
  // false for a NaN sum (a non-finite LSE): the row keeps dO . O
  if (lane == 0 && fabsf(psum - 1.f) <= kWholeRowTol) p.delta[bh * p.stat_stride + r] = pdp;
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// ACC: dK and dV are added to (or written to) the fp32 accumulators of
// attn_bwd_accumulate instead of being rounded to bf16.
template <int D, bool CAUSAL, bool ACC>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kQT * D;
  constexpr int NI = TILE * 2 / (8 * 1024);  // DMA instructions per wave per tensor and tile
  // Separate objects per buffer so that alias analysis keeps DMA writes into
  // one buffer from forcing waits on reads of the other.
  __shared__ __attribute__((aligned(1024))) __bf16 q_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 q_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 q_lds2[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 g_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 g_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 g_lds2[TILE];
  __shared__ __attribute__((aligned(1024))) float st_lds0[2 * kQT];  // [LSE*log2e | Delta] of the tile
  __shared__ __attribute__((aligned(1024))) float st_lds1[2 * kQT];
  __shared__ __attribute__((aligned(1024))) float st_lds2[2 * kQT];
  // P (bf16) handed from wave A to wave B: [step parity][pair][query block][2][lane] x 8 bf16
  __shared__ __attribute__((aligned(1024))) u32x4 xchg[2][4][2][2][64];
  __shared__ int red[2][8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const int role = wave >> 2;  // 0: S, P, dV   1: dP, dS, dK
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  // Launch order: kv heads fastest, then key blocks in the heaviest-first
  // order that the Delta pass wrote to the workspace. Workgroups are
  // dealt round-robin to the 8 XCDs, so with up to 8 kv heads each XCD keeps
  // working on the same kv head and shares its Q/dO tiles in its L2.
  const int bh = blockIdx.x;
  const int b = bh / p.hkv;
  const int hk = bh - b * p.hkv;
  const int G = p.hq / p.hkv;
  // clamped, so that a workspace without a Delta pass gives wrong sums, never a stray address
  const int ns = p.head_split;
  const int entry = (int)min((unsigned)p.order[blockIdx.y], (unsigned)(p.num_blk * ns - 1));
  const int kblk = __builtin_amdgcn_readfirstlane(entry / ns);
  const int split = __builtin_amdgcn_readfirstlane(entry - kblk * ns);
  const int k0 = kblk * 128;
  const int my_k = k0 + pair * 32 + n;
  const bool k_ok = my_k < p.seqlen;
  const int kv_stride = p.hkv * D;
  const int q_stride = p.hq * D;

  // queries that see this lane's key: [qlo, qhi)
  int qlo = 0, qhi = 0;
  if (k_ok) {
    int s0, s1;
    segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, my_k, s0, s1);
    qlo = CAUSAL ? my_k : s0;
    qhi = s1;
  }
  // Both waves of a pair hold the same keys and so take the same decisions.
  const int lo_min = __builtin_amdgcn_readfirstlane(wave_min(k_ok ? qlo : INT32_MAX));
  const int hi_max = __builtin_amdgcn_readfirstlane(wave_max(k_ok ? qhi : INT32_MIN));
  const int lo_max = __builtin_amdgcn_readfirstlane(wave_max(k_ok ? qlo : INT32_MIN));
  const int hi_min = __builtin_amdgcn_readfirstlane(wave_min(k_ok ? qhi : INT32_MAX));
  if (lane == 0) {
    red[0][wave] = lo_min;
    red[1][wave] = hi_max;
  }
  __syncthreads();
  int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    wg_lo = min(wg_lo, red[0][w]);
    wg_hi = max(wg_hi, red[1][w]);
  }
  wg_lo = __builtin_amdgcn_readfirstlane(wg_lo);
  wg_hi = __builtin_amdgcn_readfirstlane(wg_hi);
  const int tile_begin = wg_hi > wg_lo ? wg_lo / kQT : 0;
  const int tile_end = wg_hi > wg_lo ? (wg_hi + kQT - 1) / kQT : 0;
  const int ntiles = tile_end - tile_begin;
  int g_lo, g_hi;  // this workgroup's query heads of the group
  share_range(G, ns, split, g_lo, g_hi);
  g_lo = __builtin_amdgcn_readfirstlane(g_lo);
  g_hi = __builtin_amdgcn_readfirstlane(g_hi);
  const int nsteps = ntiles * (g_hi - g_lo);

  // This wave's operand (K for A, V for B) as B operands: lane (n, h) holds row my_k, d = 16t + 8h .. +7
  bf16x8 xf[KS];
  {
    const __bf16* src = role == 0 ? p.k : p.v;
    const size_t off = ((size_t)b * p.seqlen + min(my_k, p.seqlen - 1)) * kv_stride + hk * D + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) xf[t] = as_bf16x8(load16(src + off + 16 * t));
  }

  // LDS offsets: rows perm_rows(n) of a Q/dO tile (A operand of S and dP), and
  // the two transposing reads of the Q^T / dO^T fragment of query step 0.
  int qoff[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) qoff[t] = row_frag_dual<D>(lane, t);
  int trlo[DB], trhi[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    trlo[d] = tr_frag_dual<D>(lane, d, 0);
    trhi[d] = tr_frag_dual<D>(lane, d, 1);
  }
  // DMA: instruction i of wave w fills the 1 KiB at (8 i + w) KiB of a tile.
  uint32_t ld_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) ld_off[i] = dma_src_dual<D>(tile_dma_elem(i, 8, wave, lane), q_stride);
  const size_t stat_b = (size_t)b * p.hq * p.stat_stride;
  // Step order: query tiles from the last one down, the G heads of the group
  // innermost. Every workgroup of a kv head starts on the same tile, so the
  // ones running together on an XCD read the same Q/dO tiles at the same time.
  // (g, ti) of a step are carried as scalars and advanced by one per step:
  // no integer division in the loop.
  auto advance = [&](int& g, int& ti) {
    ++g;
    if (g == g_hi) {
      g = g_lo;
      --ti;
    }
  };
  auto slot_ptrs = [&](auto slot_c, __bf16*& qd, __bf16*& gd, float*& sd) {
    constexpr int sl = decltype(slot_c)::value;
    qd = sl == 0 ? q_lds0 : (sl == 1 ? q_lds1 : q_lds2);
    gd = sl == 0 ? g_lds0 : (sl == 1 ? g_lds1 : g_lds2);
    sd = sl == 0 ? st_lds0 : (sl == 1 ? st_lds1 : st_lds2);
  };
  // DMA of one step's Q and dO tiles and row statistics into buffer slot sl
  auto issue_step = [&](int g, int ti, auto slot_c) {
    const int t0 = ti * kQT;
    const int hq = hk * G + g;
    const size_t row0 = ((size_t)b * p.seqlen + t0) * q_stride + hq * D;
    const uint32_t nbytes = (uint32_t)(p.seqlen - t0) * (uint32_t)q_stride * 2u;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + row0, nbytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.dout + row0, nbytes);
    __bf16 *qd, *gd;
    float* sd;
    slot_ptrs(slot_c, qd, gd, sd);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int el = tile_dma_elem(i, 8, wave, 0);
      dma16_buf(rq, ld_off[i], qd + el);
      dma16_buf(rg, ld_off[i], gd + el);
    }
    if (wave < 2 && lane < kQT / 4) {
      // wave 0 copies LSE*log2e, wave 1 Delta: 4 floats per lane
      const float* src = (wave == 0 ? p.lse2 : p.delta) + stat_b + (size_t)hq * p.stat_stride + t0;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)(p.stat_stride - t0) * 4u);
      dma16_buf(rs, (uint32_t)lane * 16u, sd + wave * kQT);
    }
  };

  f32x16 acc[DB];  // dV^T (role A) or dK^T (role B)
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float c = p.scale_log2e, dk_mul = p.scale;
  if (p.descale_q != nullptr) {
    // fp8 inputs: scores of the codes times scale * d_q * d_k (as the fp8
    // forward computes them); dK = scale * d_q * d_v * sum dS'^T Q8
    const float dq = p.descale_q[0], dk = p.descale_k[0], dv = p.descale_v[0];
    c = p.scale * dq * dk * kLog2e;
    dk_mul = p.scale * dq * dv;
  }

  int nx_g = g_lo, nx_ti = tile_end - 1;  // head and query tile of the next step to load
  if (nsteps > 0) {
    issue_step(nx_g, nx_ti, std::integral_constant<int, 0>{});
    advance(nx_g, nx_ti);
  }
  wait_dma();
  __syncthreads();

  // Every pair runs every step of the workgroup's range: a step that a pair
  // cannot see is fully masked (P = 0). With 64-query tiles and 128-key
  // workgroups that costs at most the first two steps of a causal range,
  // and it keeps the loop free of per-wave branches around the barriers.
  //
  // Wave B runs one step behind wave A, so the two are independent within a
  // step and one barrier per step suffices:
  //   step j: A: S(j) = Q(j) K^T, P(j) -> exchange slot j % 2, dV^T += dO(j)^T P(j)
  //           B: dP(j-1) = dO(j-1) V^T, dS(j-1) with P(j-1), dK^T += Q(j-1)^T dS(j-1)
  // Tiles therefore live for two steps (three buffer slots; the next step's
  // tiles load into the third), the exchange for two (two slots). P goes
  // through LDS as bf16; dS is rounded to bf16 for its MFMA anyway. Slots are
  // compile-time: the loop over the nsteps + 1 barrier steps is unrolled by 6.
  const int nbar = nsteps > 0 ? nsteps + 1 : 0;
  auto steps6 = [&](auto body) {
    for (int s0 = 0; s0 < nbar; s0 += 6) {
      body(s0, std::integral_constant<int, 0>{});
      if (s0 + 1 < nbar) body(s0 + 1, std::integral_constant<int, 1>{});
      if (s0 + 2 < nbar) body(s0 + 2, std::integral_constant<int, 2>{});
      if (s0 + 3 < nbar) body(s0 + 3, std::integral_constant<int, 3>{});
      if (s0 + 4 < nbar) body(s0 + 4, std::integral_constant<int, 4>{});
      if (s0 + 5 < nbar) body(s0 + 5, std::integral_constant<int, 5>{});
    }
  };
  auto prefetch = [&](int step, auto r_c) {
    constexpr int r = decltype(r_c)::value;
    if (step + 1 < nsteps) {
      issue_step(nx_g, nx_ti, std::integral_constant<int, (r + 1) % 3>{});
      advance(nx_g, nx_ti);
    }
  };
  // out[qb] += (rows qb*32 .. qb*32+31 of a Q or dO tile) x (this wave's K or
  // V)^T. The two 32-row chains alternate, and the LDS operands of step t + 2
  // are read before the MFMAs of step t, so the read latency overlaps MFMAs.
  auto rows_times_x = [&](const __bf16* tile, f32x16 (&out)[2]) {
    bf16x8 a[3][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) a[t][qb] = lds_read_b128(tile, qoff[t] + qb * 32 * D);
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t + 2 < KS) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) a[(t + 2) % 3][qb] = lds_read_b128(tile, qoff[t + 2] + qb * 32 * D);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) out[qb] = mfma32(a[t % 3][qb], xf[t], out[qb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dV^T += dO^T P (role A) or dK^T += Q^T dS (role B) for one step's tile:
  // the transposed fragments of query step u + 1 are read before the MFMAs
  // of step u.
  auto tr_times = [&](const __bf16* tile, const bf16x8 (&pk)[4]) {
    bf16x8 fr[2][DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) fr[0][d] = tr_read2(tile, trlo[d], trhi[d]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < 3) {
#pragma unroll
        for (int d = 0; d < DB; ++d)
          fr[(u + 1) & 1][d] = tr_read2(tile, trlo[d] + 16 * (u + 1) * D, trhi[d] + 16 * (u + 1) * D);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d) acc[d] = mfma32(fr[u & 1][d], pk[u], acc[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The two waves of a SIMD (A and B of one pair) alternate between the
  // matrix pipe and the vector ALU within each barrier step:
  //   A: S(j) and dV^T += dO(j-1)^T P(j-1)  [MFMA]  then P(j) = exp2(...)    [VALU]
  //   B: dS(j-1) = P(j-1) (dP(j-1) - Delta) [VALU]  then dK^T += Q(j-1)^T dS(j-1), dP(j) [MFMA]
  // so while one wave computes exponentials or dS the other keeps the matrix
  // pipe busy. A carries P(j) and B carries dP(j) in registers into the next
  // step; B reads P(j-1) from the exchange slot A wrote in step j - 1.
  if (role == 0) {
    int cur_g = g_lo, cur_ti = tile_end - 1;
    bf16x8 pk[4];  // P of the previous step (bf16)
    auto body_a = [&](int step, auto r_c) {
      constexpr int r = decltype(r_c)::value;
      prefetch(step, r_c);
      __bf16 *qs, *gs;
      float* st;
      slot_ptrs(std::integral_constant<int, r % 3>{}, qs, gs, st);
      f32x16 sc[2] = {f32x16{}, f32x16{}};
      if (step < nsteps) rows_times_x(qs, sc);
      if (step > 0) {
        __bf16 *qp, *gp;
        float* sp;
        slot_ptrs(std::integral_constant<int, (r + 2) % 3>{}, qp, gp, sp);
        tr_times(gp, pk);
      }
      if (step < nsteps) {
        const int t0 = cur_ti * kQT;
        const bool full = (t0 >= lo_max) && (t0 + kQT <= hi_min);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x16& s = sc[qb];
          // C rows of this lane: queries qb*32 + c_key(r, h), two runs of 8
          const float* l4 = st + qb * 32 + 8 * h;
          const f32x4 la = lds_load16<f32x4>(l4), lb = lds_load16<f32x4>(l4 + 4);
          const f32x4 lc = lds_load16<f32x4>(l4 + 16), ld = lds_load16<f32x4>(l4 + 20);
          float pr[16];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pr[e] = fast_exp2(__builtin_fmaf(s[e], c, -la[e]));
            pr[4 + e] = fast_exp2(__builtin_fmaf(s[4 + e], c, -lb[e]));
            pr[8 + e] = fast_exp2(__builtin_fmaf(s[8 + e], c, -lc[e]));
            pr[12 + e] = fast_exp2(__builtin_fmaf(s[12 + e], c, -ld[e]));
          }
          if (!full) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int qq = t0 + qb * 32 + c_key(rr, h);
              pr[rr] = (qq < qlo || qq >= qhi) ? 0.f : pr[rr];
            }
          }
          pk[2 * qb] = pack_bf16(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
          pk[2 * qb + 1] = pack_bf16(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
          xchg[r % 2][pair][qb][0][lane] = __builtin_bit_cast(u32x4, pk[2 * qb]);
          xchg[r % 2][pair][qb][1][lane] = __builtin_bit_cast(u32x4, pk[2 * qb + 1]);
        }
        advance(cur_g, cur_ti);
      }
      wait_dma();
      __syncthreads();
    };
    steps6(body_a);
  } else {
    f32x16 dp[2];  // dP of the previous step
    auto body_b = [&](int step, auto r_c) {
      constexpr int r = decltype(r_c)::value;
      prefetch(step, r_c);
      if (step > 0) {
        // tiles and exchange slot of step - 1
        __bf16 *qs, *gs;
        float* st;
        slot_ptrs(std::integral_constant<int, (r + 2) % 3>{}, qs, gs, st);
        constexpr int xs = (r + 1) % 2;
        bf16x8 db[4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          // dS = P (dP - Delta), P widened from the bf16 exchange
          const float* d4 = st + kQT + qb * 32 + 8 * h;
          const f32x4 da = lds_load16<f32x4>(d4), dd = lds_load16<f32x4>(d4 + 4);
          const f32x4 dc = lds_load16<f32x4>(d4 + 16), de = lds_load16<f32x4>(d4 + 20);
          const u32x4 w0 = xchg[xs][pair][qb][0][lane], w1 = xchg[xs][pair][qb][1][lane];
          auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
          auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
          float dsv[16];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            dsv[2 * e] = lo(w0[e]) * (dp[qb][2 * e] - da[2 * e]);
            dsv[2 * e + 1] = hi(w0[e]) * (dp[qb][2 * e + 1] - da[2 * e + 1]);
            dsv[4 + 2 * e] = lo(w0[2 + e]) * (dp[qb][4 + 2 * e] - dd[2 * e]);
            dsv[5 + 2 * e] = hi(w0[2 + e]) * (dp[qb][5 + 2 * e] - dd[2 * e + 1]);
            dsv[8 + 2 * e] = lo(w1[e]) * (dp[qb][8 + 2 * e] - dc[2 * e]);
            dsv[9 + 2 * e] = hi(w1[e]) * (dp[qb][9 + 2 * e] - dc[2 * e + 1]);
            dsv[12 + 2 * e] = lo(w1[2 + e]) * (dp[qb][12 + 2 * e] - de[2 * e]);
            dsv[13 + 2 * e] = hi(w1[2 + e]) * (dp[qb][13 + 2 * e] - de[2 * e + 1]);
          }
          db[2 * qb] = pack_bf16(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
          db[2 * qb + 1] = pack_bf16(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
        }
        tr_times(qs, db);
      }
      if (step < nsteps) {
        __bf16 *qs, *gs;
        float* st;
        slot_ptrs(std::integral_constant<int, r % 3>{}, qs, gs, st);
        dp[0] = f32x16{};
        dp[1] = f32x16{};
        rows_times_x(gs, dp);
      }
      wait_dma();
      __syncthreads();
    };
    steps6(body_b);
  }

  if (k_ok) {
    const float mul = role == 0 ? 1.0f : dk_mul;
    const size_t row = ((size_t)b * p.seqlen + my_k) * kv_stride + hk * D;
    if (ACC && ns == 1) {
      // fp32 accumulators: added to (or written when accumulate = 0)
      float* dst = (role == 0 ? p.dv_acc : p.dk_acc) + row;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* cell = reinterpret_cast<f32x4*>(dst + 32 * d + 8 * g + 4 * h);
          f32x4 w = p.accumulate ? *cell : f32x4{};
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] += acc[d][4 * g + e] * mul;
          *cell = w;
        }
    } else if (ns == 1) {
      __bf16* dst = (role == 0 ? p.dv : p.dk) + row;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[d][4 * g + e] * mul);
          *reinterpret_cast<bf16x4*>(dst + 32 * d + 8 * g + 4 * h) = w;
        }
    } else {
      // fp32 partial of this share of the heads: part[dK | dV][split][b][s][hk][d]
      const size_t plane = (size_t)p.batch * p.seqlen * kv_stride;
      float* dst = p.part + (size_t)(role == 0 ? 1 : 0) * ns * plane + (size_t)split * plane + row;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[d][4 * g + e] * mul;
          *reinterpret_cast<f32x4*>(dst + 32 * d + 8 * g + 4 * h) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV = sum of the head-share partials, rounded to bf16 (head_split > 1),
// or added to the fp32 accumulators of attn_bwd_accumulate
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dkdv_reduce_kernel(BwdParams p) {
  const size_t plane = (size_t)p.batch * p.seqlen * p.hkv * p.head_dim;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  const int ns = p.head_split;
#pragma unroll
  for (int t = 0; t < 2; ++t) {  // 0: dK, 1: dV
    const float* src = p.part + (size_t)t * ns * plane + i;
    f32x4 sum = *reinterpret_cast<const f32x4*>(src);
    for (int sp = 1; sp < ns; ++sp) sum += *reinterpret_cast<const f32x4*>(src + (size_t)sp * plane);
    if (p.dk_acc != nullptr) {
      f32x4* cell = reinterpret_cast<f32x4*>((t == 0 ? p.dk_acc : p.dv_acc) + i);
      *cell = p.accumulate ? *cell + sum : sum;
      continue;
    }
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (__bf16)sum[e];
    *reinterpret_cast<bf16x4*>((t == 0 ? p.dk : p.dv) + i) = w;
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// ACC: dQ is added to (or written to) the fp32 accumulator of
// attn_bwd_accumulate instead of being rounded to bf16.
// WAVES waves of 32 queries per workgroup: 4 (128-query blocks, two
// workgroups per CU) or 8 (256-query blocks, one per CU sharing each K/V
// tile); bwd_dq_block_waves() picks one.
template <int D, bool CAUSAL, bool ACC, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kKT * D;
  constexpr int NI = TILE * 2 / (WAVES * 1024);
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[TILE];  // dual layout: rows and K^T reads
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[TILE];  // row reads only
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[TILE];
  __shared__ int red[2][WAVES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int hq = bh - b * p.hq;
  const int hk = hq / (p.hq / p.hkv);
  const int nks = p.key_split;
  const int qentry =
      (int)min((unsigned)p.order[p.num_blk * p.head_split + blockIdx.y], (unsigned)(p.num_dq_blk * nks - 1));
  const int qblk = __builtin_amdgcn_readfirstlane(qentry / nks);
  const int ksplit = __builtin_amdgcn_readfirstlane(qentry - qblk * nks);
  const int my_q = qblk * (32 * WAVES) + wave * 32 + n;
  const bool q_ok = my_q < p.seqlen;
  const int q_stride = p.hq * D;
  const int kv_stride = p.hkv * D;
  const __bf16* kg = p.k + (size_t)b * p.seqlen * kv_stride + hk * D;
  const __bf16* vg = p.v + (size_t)b * p.seqlen * kv_stride + hk * D;

  int kstart = 0, kend = 0;
  if (q_ok) {
    int s0, s1;
    segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, my_q, s0, s1);
    kstart = s0;
    kend = CAUSAL ? my_q + 1 : s1;
  }
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
  for (int w = 0; w < WAVES; ++w) {
    wg_lo = min(wg_lo, red[0][w]);
    wg_hi = max(wg_hi, red[1][w]);
  }
  wg_lo = __builtin_amdgcn_readfirstlane(wg_lo);
  wg_hi = __builtin_amdgcn_readfirstlane(wg_hi);
  // this workgroup's share of the block's visible key tiles
  int tile_begin = wg_hi > wg_lo ? wg_lo / kKT : 0;
  int tile_end = wg_hi > wg_lo ? (wg_hi + kKT - 1) / kKT : 0;
  {
    int lo, hi;
    share_range(tile_end - tile_begin, nks, ksplit, lo, hi);
    tile_end = __builtin_amdgcn_readfirstlane(tile_begin + hi);
    tile_begin = __builtin_amdgcn_readfirstlane(tile_begin + lo);
  }

  bf16x8 qf[KS], gf[KS];
  {
    const size_t off = ((size_t)b * p.seqlen + min(my_q, p.seqlen - 1)) * q_stride + hq * D + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      qf[t] = as_bf16x8(load16(p.q + off + 16 * t));
      gf[t] = as_bf16x8(load16(p.dout + off + 16 * t));
    }
  }
  const size_t so = ((size_t)b * p.hq + hq) * p.stat_stride;
  // rows past the end: P = exp2(-inf) = 0, so nothing from them is non-finite
  const float lse2 = q_ok ? p.lse2[so + my_q] : INFINITY;
  const float dlt = q_ok ? p.delta[so + my_q] : 0.f;

  int koff[KS], voff[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    koff[t] = row_frag_dual<D>(lane, t);
    voff[t] = row_frag_b128<D>(lane, t);
  }
  int ktlo[DB], kthi[DB];  // K^T fragment of key step 0
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    ktlo[d] = tr_frag_dual<D>(lane, d, 0);
    kthi[d] = tr_frag_dual<D>(lane, d, 1);
  }
  uint32_t ld_koff[NI], ld_voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = tile_dma_elem(i, WAVES, wave, lane);
    ld_koff[i] = dma_src_dual<D>(e, kv_stride);
    ld_voff[i] = dma_src_b128<D>(e, kv_stride);
  }
  auto issue_tile = [&](int t0, auto buf_c) {
    __bf16* kd = decltype(buf_c)::value ? k_lds1 : k_lds0;
    __bf16* vd = decltype(buf_c)::value ? v_lds1 : v_lds0;
    const uint32_t nbytes = (uint32_t)(p.seqlen - t0) * (uint32_t)kv_stride * 2u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)t0 * kv_stride, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)t0 * kv_stride, nbytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int el = tile_dma_elem(i, WAVES, wave, 0);
      dma16_buf(rk, ld_koff[i], kd + el);
      dma16_buf(rv, ld_voff[i], vd + el);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float c = p.scale_log2e, dq_mul = p.scale;
  if (p.descale_q != nullptr) {
    // fp8 inputs: dQ = scale * d_k * d_v * sum dS' K8
    const float dq = p.descale_q[0], dk = p.descale_k[0], dv = p.descale_v[0];
    c = p.scale * dq * dk * kLog2e;
    dq_mul = p.scale * dk * dv;
  }

  if (tile_begin < tile_end) issue_tile(tile_begin * kKT, std::integral_constant<int, 0>{});
  wait_dma();
  __syncthreads();

  auto tile_body = [&](int it, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    const int t0 = it * kKT;
    if (it + 1 < tile_end) issue_tile(t0 + kKT, std::integral_constant<int, cur ^ 1>{});
    if ((t0 < hi_max) && (t0 + kKT > lo_min)) {
      const bool full = (t0 >= lo_max) && (t0 + kKT <= hi_min);
      const __bf16* ks = cur ? k_lds1 : k_lds0;
      const __bf16* vs = cur ? v_lds1 : v_lds0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S and dP chains alternate; LDS operands are read two steps ahead
        f32x16 s = f32x16{}, dp = f32x16{};
        {
          bf16x8 ka[3], va[3];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            ka[t] = lds_read_b128(ks, koff[t] + kb * 32 * D);
            va[t] = lds_read_b128(vs, voff[t] + kb * 32 * D);
          }
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            if (t + 2 < KS) {
              ka[(t + 2) % 3] = lds_read_b128(ks, koff[t + 2] + kb * 32 * D);
              va[(t + 2) % 3] = lds_read_b128(vs, voff[t + 2] + kb * 32 * D);
            }
            s = mfma32(ka[t % 3], qf[t], s);
            dp = mfma32(va[t % 3], gf[t], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // K^T fragments of the first 16 keys, read while the exponentials run
        const int o = (kb * 32) * D;
        bf16x8 f0[DB], f1[DB];
#pragma unroll
        for (int d = 0; d < DB; ++d) f0[d] = tr_read2(ks, ktlo[d] + o, kthi[d] + o);
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          dsv[r] = pr * (dp[r] - dlt);
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t0 + kb * 32 + c_key(r, h);
            dsv[r] = (key < kstart || key >= kend) ? 0.f : dsv[r];
          }
        }
        const bf16x8 d0 = pack_bf16(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        const bf16x8 d1 = pack_bf16(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
        // dQ^T += K^T dS^T
#pragma unroll
        for (int d = 0; d < DB; ++d) f1[d] = tr_read2(ks, ktlo[d] + o + 16 * D, kthi[d] + o + 16 * D);
#pragma unroll
        for (int d = 0; d < DB; ++d) acc[d] = mfma32(f0[d], d0, acc[d]);
#pragma unroll
        for (int d = 0; d < DB; ++d) acc[d] = mfma32(f1[d], d1, acc[d]);
      }
    }
    wait_dma();
    __syncthreads();
  };

  for (int it = tile_begin; it < tile_end; it += 2) {
    tile_body(it, std::integral_constant<int, 0>{});
    if (it + 1 < tile_end) tile_body(it + 1, std::integral_constant<int, 1>{});
  }

  if (q_ok) {
    const size_t roff = ((size_t)b * p.seqlen + my_q) * q_stride + hq * D;
    if (ACC && nks == 1) {
      // fp32 accumulator: added to (or written when accumulate = 0)
      float* row = p.dq_acc + roff;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* cell = reinterpret_cast<f32x4*>(row + 32 * d + 8 * g + 4 * h);
          f32x4 w = p.accumulate ? *cell : f32x4{};
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] += acc[d][4 * g + e] * dq_mul;
          *cell = w;
        }
    } else if (nks == 1) {
      __bf16* row = p.dq + roff;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[d][4 * g + e] * dq_mul);
          *reinterpret_cast<bf16x4*>(row + 32 * d + 8 * g + 4 * h) = w;
        }
    } else {
      // fp32 partial of this share of the key tiles: dq_part[split][b][s][hq][d]
      float* row = p.dq_part + (size_t)ksplit * p.batch * p.seqlen * q_stride + roff;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[d][4 * g + e] * dq_mul;
          *reinterpret_cast<f32x4*>(row + 32 * d + 8 * g + 4 * h) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ = sum of the key-share partials, rounded to bf16 (key_split > 1), or
// added to the fp32 accumulator of attn_bwd_accumulate
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_bwd_dq_reduce_kernel(BwdParams p) {
  const size_t plane = (size_t)p.batch * p.seqlen * p.hq * p.head_dim;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= plane) return;
  const float* src = p.dq_part + i;
  f32x4 sum = *reinterpret_cast<const f32x4*>(src);
  for (int sp = 1; sp < p.key_split; ++sp) sum += *reinterpret_cast<const f32x4*>(src + (size_t)sp * plane);
  if (p.dq_acc != nullptr) {
    f32x4* cell = reinterpret_cast<f32x4*>(p.dq_acc + i);
    *cell = p.accumulate ? *cell + sum : sum;
    return;
  }
  bf16x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (__bf16)sum[e];
  *reinterpret_cast<bf16x4*>(p.dq + i) = w;
}

// ---------------------------------------------------------------------------
// E4M3FN code -> bf16, exactly: a code is (-1)^s 2^(e-7) (1 + m/8) for
// exponent field e > 0 and (-1)^s 2^-6 (m/8) for e = 0; e = 15, m = 7 is NaN.
// Every such value has at most 4 significant bits and an exponent in
// [-9, 8], so bf16 holds it exactly. 16 codes per thread.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __bf16 e4m3_to_bf16(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u) {
    v = __builtin_nanf("");
  } else if (e == 0u) {
    v = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // 2^(e-7) (1 + m/8)
  }
  return (__bf16)((b & 0x80u) ? -v : v);
}

__global__ __launch_bounds__(256) void attn_widen_fp8_kernel(const uint8_t* src, __bf16* dst, size_t n) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= n) return;
  if (i + 16 <= n) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + i);
    bf16x8 lo, hi;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lo[k] = e4m3_to_bf16((w[k / 4] >> (8 * (k % 4))) & 0xFFu);
      hi[k] = e4m3_to_bf16((w[2 + k / 4] >> (8 * (k % 4))) & 0xFFu);
    }
    *reinterpret_cast<bf16x8*>(dst + i) = lo;
    *reinterpret_cast<bf16x8*>(dst + i + 8) = hi;
  } else {
    for (size_t k = i; k < n; ++k) dst[k] = e4m3_to_bf16(src[k]);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdParams& p_in, unsigned phases, hipStream_t stream) {
  BwdParams q = p_in;
  q.num_blk = (q.seqlen + 127) / 128;
  if (q.dq_waves != 8) q.dq_waves = 4;
  q.num_dq_blk = (q.seqlen + 32 * q.dq_waves - 1) / (32 * q.dq_waves);
  if (phases & kBwdDelta) {
    constexpr int RPW = 256 / (D / 8) * kDeltaRows;
    const long nrows = (long)q.batch * q.seqlen * q.hq;
    const long nstat = (nrows + RPW - 1) / RPW;
    const long npadwg = ((long)q.batch * q.hq * (q.stat_stride - q.seqlen) + 255) / 256;
    const long norder =
        (q.num_blk * (long)q.head_split + 255) / 256 + (q.num_dq_blk * (long)q.key_split + 255) / 256;
    dim3 grid((unsigned)(nstat + npadwg + norder));
    hipLaunchKernelGGL((attn_bwd_delta_kernel<D, CAUSAL>), grid, dim3(256), 0, stream, q);
    // rows with fewer than 64 visible keys: none for a dense non-causal call with S >= 64
    if (CAUSAL || q.cu_seqlens != nullptr || q.seqlen < kFewKeyLimit) {
      const int nseg = q.cu_seqlens != nullptr ? q.num_seqs : 1;
      const dim3 fgrid((unsigned)nseg * kFewBlocksB, q.hq, q.batch);
      hipLaunchKernelGGL((attn_bwd_delta_fewkeys_kernel<D, CAUSAL>), fgrid, dim3(256), 0, stream, q);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDkDv) {
    dim3 grid(q.batch * q.hkv, q.num_blk * q.head_split);
    if (q.dk_acc != nullptr) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, true>), grid, dim3(512), 0, stream, q);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, false>), grid, dim3(512), 0, stream, q);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (q.head_split > 1) {
      const size_t quads = (size_t)q.batch * q.seqlen * q.hkv * D / 4;
      hipLaunchKernelGGL(attn_bwd_dkdv_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, q);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (phases & kBwdDq) {
    dim3 grid(q.batch * q.hq, q.num_dq_blk * q.key_split);
    if (q.dq_waves == 8) {
      if (q.dq_acc != nullptr) {
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, true, 8>), grid, dim3(512), 0, stream, q);
      } else {
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, false, 8>), grid, dim3(512), 0, stream, q);
      }
    } else if (q.dq_acc != nullptr) {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, true, 4>), grid, dim3(256), 0, stream, q);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, false, 4>), grid, dim3(256), 0, stream, q);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (q.key_split > 1) {
      const size_t quads = (size_t)q.batch * q.seqlen * q.hq * D / 4;
      hipLaunchKernelGGL(attn_bwd_dq_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, q);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t run_widen_fp8(const uint8_t* src, __bf16* dst, size_t n, hipStream_t stream) {
  const size_t threads = (n + 15) / 16;
  hipLaunchKernelGGL(attn_widen_fp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

hipError_t run_bwd(const BwdParams& p, unsigned phases, hipStream_t stream) {
  if (p.head_dim == 128) {
    return p.causal ? launch_bwd<128, true>(p, phases, stream) : launch_bwd<128, false>(p, phases, stream);
  }
  return p.causal ? launch_bwd<64, true>(p, phases, stream) : launch_bwd<64, false>(p, phases, stream);
}

#ifdef ATTN_DEBUG
hipError_t lds_faults_bwd(unsigned int* out) { return take_lds_fault_word(out); }
#endif

}  // namespace mi355attn
