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
// Split into two passes so that nothing is accumulated with atomics:
//   * dK/dV: one workgroup per (b, h_kv, 32*NW keys); each wave keeps 32 keys
//     of K and V in VGPRs and accumulates dK^T, dV^T over every query head of
//     the GQA group and every visible Q tile (so the group sum needs no
//     reduction across workgroups);
//   * dQ: one workgroup per (b, h_q, 32*NW queries), the forward's layout:
//     Q and dO stay in VGPRs, K and V tiles stream through LDS.
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

constexpr int kTile = 64;  // rows of the streamed tiles (queries or keys)

// One layout for tiles read both with 16-byte reads (rows through perm_rows)
// and with transposing reads (4 consecutive rows): the chunk XOR spreads
// 16 consecutive rows over 16 chunks and 4 consecutive rows over 4 chunk groups.
template <int D>
__device__ __forceinline__ int swz_dual(int row, int chunk) {
  if constexpr (D == 128) {
    return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    return chunk ^ (((row & 3) << 1) | ((row >> 2) & 1));
  }
}
template <int D>
__device__ __forceinline__ int off_dual(int row, int chunk) { return row * D + swz_dual<D>(row, chunk) * 8; }
template <int D>
__device__ __forceinline__ int off_dual_unit(int row, int unit) {
  return row * D + swz_dual<D>(row, unit >> 1) * 8 + (unit & 1) * 4;
}

// X^T fragment from a dual-layout tile (see tr_fragment in attn_device.h).
template <int D>
__device__ __forceinline__ bf16x8 tr_fragment_dual(const __bf16* tile, int row0, int col0, int lane) {
  const int r = row0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int unit = (col0 >> 2) + 4 * ((lane >> 4) & 1) + (lane & 3);
  const bf16x4 lo = lds_read_tr(tile, off_dual_unit<D>(r, unit));
  const bf16x4 hi = lds_read_tr(tile, off_dual_unit<D>(r + 4, unit));
  bf16x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

// ---------------------------------------------------------------------------
// Delta_i = dO_i . O_i (fp32), [B, Hq, S]
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / LPR;  // index into [B, S, Hq]
  const long nrows = (long)p.batch * p.seqlen * p.hq;
  const int sub = tid % LPR;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = load16(p.o + row * D + sub * 8);
    const u32x4 g = load16(p.dout + row * D + sub * 8);
    const bf16x8 av = as_bf16x8(a), gv = as_bf16x8(g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)av[e] * (float)gv[e];
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < nrows && sub == 0) {
    const long hq = row % p.hq;
    const long bs = row / p.hq;
    const long i = bs % p.seqlen;
    const long b = bs / p.seqlen;
    p.delta[(b * p.hq + hq) * p.seqlen + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <int D, int NW>
struct QTileLoader {
  static constexpr int kThreads = NW * 64;
  static constexpr int kChunks = kTile * D / 8;
  static constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  u32x4 q[kPer], g[kPer];
  float lse2, dlt;  // one row statistic per thread (threads < kTile)

  __device__ __forceinline__ void load(const BwdParams& p, int b, int hq, int t0, int tid) {
    const int q_stride = p.hq * D;
    const __bf16* qg = p.q + (size_t)b * p.seqlen * q_stride + hq * D;
    const __bf16* gg = p.dout + (size_t)b * p.seqlen * q_stride + hq * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int r = t0 + row;
      const bool ok = (idx < kChunks) && r < p.seqlen;
      const size_t off = (size_t)(ok ? r : 0) * q_stride + ch * 8;
      q[i] = load16_pred(qg + off, ok);
      g[i] = load16_pred(gg + off, ok);
    }
    if (tid < kTile) {
      const int r = t0 + tid;
      const size_t so = ((size_t)b * p.hq + hq) * p.seqlen;
      const bool ok = r < p.seqlen;
      lse2 = ok ? p.lse[so + r] * kLog2e : INFINITY;
      dlt = ok ? p.delta[so + r] : 0.f;
    }
  }
  __device__ __forceinline__ void store(__bf16* qs, __bf16* gs, float* ls, float* ds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < kChunks) {
        const int row = idx / (D / 8);
        const int ch = idx % (D / 8);
        lds_store16(qs, off_dual<D>(row, ch), q[i]);
        lds_store16(gs, off_dual<D>(row, ch), g[i]);
      }
    }
    if (tid < kTile) {
      ls[tid] = lse2;
      ds[tid] = dlt;
    }
  }
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int BK = 32 * NW;  // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) __bf16 g_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) float l_lds[2][kTile];
  __shared__ __attribute__((aligned(16))) float d_lds[2][kTile];
  __shared__ int red[2][NW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hkv;
  const int hk = bh - b * p.hkv;
  const int G = p.hq / p.hkv;
  const int kblk = blockIdx.y;
  const int k0 = kblk * BK;
  const int my_k = k0 + wave * 32 + n;
  const bool k_ok = my_k < p.seqlen;
  const int kv_stride = p.hkv * D;

  // queries that see this lane's key: [qlo, qhi)
  int qlo = 0, qhi = 0;
  if (k_ok) {
    int s0, s1;
    segment_of(p.cu_seqlens, p.num_seqs, p.seqlen, my_k, s0, s1);
    qlo = CAUSAL ? my_k : s0;
    qhi = s1;
  }
  const int lo_min = wave_min(k_ok ? qlo : INT32_MAX);
  const int hi_max = wave_max(k_ok ? qhi : INT32_MIN);
  const int lo_max = wave_max(k_ok ? qlo : INT32_MIN);
  const int hi_min = wave_min(k_ok ? qhi : INT32_MAX);
  if (lane == 0) {
    red[0][wave] = lo_min;
    red[1][wave] = hi_max;
  }
  __syncthreads();
  int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wg_lo = min(wg_lo, red[0][w]);
    wg_hi = max(wg_hi, red[1][w]);
  }
  const int tile_begin = wg_hi > wg_lo ? wg_lo / kTile : 0;
  const int tile_end = wg_hi > wg_lo ? (wg_hi + kTile - 1) / kTile : 0;
  const int ntiles = tile_end - tile_begin;
  const int nsteps = ntiles * G;

  // K and V slices of this wave as B operands: lane (n, h) holds row my_k, d = 16t + 8h .. +7
  bf16x8 kf[KS], vf[KS];
  {
    const size_t off = ((size_t)b * p.seqlen + (k_ok ? my_k : 0)) * kv_stride + hk * D + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      kf[t] = as_bf16x8(load16_pred(p.k + off + 16 * t, k_ok));
      vf[t] = as_bf16x8(load16_pred(p.v + off + 16 * t, k_ok));
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float c = p.scale_log2e;

  QTileLoader<D, NW> ld;
  if (nsteps > 0) {
    ld.load(p, b, hk * G, tile_begin * kTile, tid);
    ld.store(q_lds[0], g_lds[0], l_lds[0], d_lds[0], tid);
  }
  __syncthreads();

  const int qrow = perm_rows(n);
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const int it = tile_begin + step % ntiles;
    const int t0 = it * kTile;
    const bool more = step + 1 < nsteps;
    if (more) {
      const int nstep = step + 1;
      ld.load(p, b, hk * G + nstep / ntiles, (tile_begin + nstep % ntiles) * kTile, tid);
    }
    const bool any = (t0 < hi_max) && (t0 + kTile > lo_min);
    if (any) {
      const bool full = (t0 >= lo_max) && (t0 + kTile <= hi_min);
      const __bf16* qs = q_lds[cur];
      const __bf16* gs = g_lds[cur];
      const float* ls = l_lds[cur];
      const float* dsl = d_lds[cur];
      bf16x8 pb[4], db[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const bf16x8 a = lds_read_b128(qs, off_dual<D>(qb * 32 + qrow, 2 * t + h));
          s = mfma32(a, kf[t], s);
        }
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const bf16x8 a = lds_read_b128(gs, off_dual<D>(qb * 32 + qrow, 2 * t + h));
          dp = mfma32(a, vf[t], dp);
        }
        // rows of this lane: queries qb*32 + c_key(r, h): two runs of 8
        const f32x4* l4 = reinterpret_cast<const f32x4*>(ls + qb * 32 + 8 * h);
        const f32x4* d4 = reinterpret_cast<const f32x4*>(dsl + qb * 32 + 8 * h);
        float pr[16], dsv[16];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 la = l4[4 * half], lb = l4[4 * half + 1];
          const f32x4 da = d4[4 * half], dd = d4[4 * half + 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = 8 * half + e, r1 = 8 * half + 4 + e;
            pr[r0] = fast_exp2(__builtin_fmaf(s[r0], c, -la[e]));
            pr[r1] = fast_exp2(__builtin_fmaf(s[r1], c, -lb[e]));
            dsv[r0] = pr[r0] * (dp[r0] - da[e]);
            dsv[r1] = pr[r1] * (dp[r1] - dd[e]);
          }
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qq = t0 + qb * 32 + c_key(r, h);
            if (qq < qlo || qq >= qhi) {
              pr[r] = 0.f;
              dsv[r] = 0.f;
            }
          }
        }
        pb[2 * qb] = pack_bf16(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
        pb[2 * qb + 1] = pack_bf16(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
        db[2 * qb] = pack_bf16(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        db[2 * qb + 1] = pack_bf16(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const bf16x8 ag = tr_fragment_dual<D>(gs, 16 * u, 32 * d, lane);
          dv[d] = mfma32(ag, pb[u], dv[d]);
          const bf16x8 aq = tr_fragment_dual<D>(qs, 16 * u, 32 * d, lane);
          dk[d] = mfma32(aq, db[u], dk[d]);
        }
    }
    if (more) ld.store(q_lds[cur ^ 1], g_lds[cur ^ 1], l_lds[cur ^ 1], d_lds[cur ^ 1], tid);
    __syncthreads();
  }

  if (k_ok) {
    const size_t off = ((size_t)b * p.seqlen + my_k) * kv_stride + hk * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (__bf16)(dk[d][4 * g + e] * p.scale);
          wv[e] = (__bf16)(dv[d][4 * g + e]);
        }
        *reinterpret_cast<bf16x4*>(p.dk + off + 32 * d + 8 * g + 4 * h) = wk;
        *reinterpret_cast<bf16x4*>(p.dv + off + 32 * d + 8 * g + 4 * h) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int NW>
struct KVTileLoader {
  static constexpr int kThreads = NW * 64;
  static constexpr int kChunks = kTile * D / 8;
  static constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  u32x4 k[kPer], v[kPer];

  __device__ __forceinline__ void load(const __bf16* kg, const __bf16* vg, int row_stride, int t0, int seqlen,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int g = t0 + row;
      const bool ok = (idx < kChunks) && g < seqlen;
      const size_t off = (size_t)(ok ? g : 0) * row_stride + ch * 8;
      k[i] = load16_pred(kg + off, ok);
      v[i] = load16_pred(vg + off, ok);
    }
  }
  __device__ __forceinline__ void store(__bf16* ks, __bf16* vs, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < kChunks) {
        const int row = idx / (D / 8);
        const int ch = idx % (D / 8);
        lds_store16(ks, off_dual<D>(row, ch), k[i]);
        lds_store16(vs, off_b128<D>(row, ch), v[i]);
      }
    }
  }
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kTile * D];
  __shared__ int red[2][NW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int hq = bh - b * p.hq;
  const int hk = hq / (p.hq / p.hkv);
  const int qblk = p.num_blk - 1 - (int)blockIdx.y;
  const int my_q = qblk * BM + wave * 32 + n;
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
  const int lo_min = wave_min(q_ok ? kstart : INT32_MAX);
  const int hi_max = wave_max(q_ok ? kend : INT32_MIN);
  const int lo_max = wave_max(q_ok ? kstart : INT32_MIN);
  const int hi_min = wave_min(q_ok ? kend : INT32_MAX);
  if (lane == 0) {
    red[0][wave] = lo_min;
    red[1][wave] = hi_max;
  }
  __syncthreads();
  int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wg_lo = min(wg_lo, red[0][w]);
    wg_hi = max(wg_hi, red[1][w]);
  }
  const int tile_begin = wg_hi > wg_lo ? wg_lo / kTile : 0;
  const int tile_end = wg_hi > wg_lo ? (wg_hi + kTile - 1) / kTile : 0;

  bf16x8 qf[KS], gf[KS];
  {
    const size_t off = ((size_t)b * p.seqlen + (q_ok ? my_q : 0)) * q_stride + hq * D + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      qf[t] = as_bf16x8(load16_pred(p.q + off + 16 * t, q_ok));
      gf[t] = as_bf16x8(load16_pred(p.dout + off + 16 * t, q_ok));
    }
  }
  const size_t so = ((size_t)b * p.hq + hq) * p.seqlen;
  const float lse2 = q_ok ? p.lse[so + my_q] * kLog2e : INFINITY;
  const float dlt = q_ok ? p.delta[so + my_q] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  const float c = p.scale_log2e;

  KVTileLoader<D, NW> ld;
  if (tile_begin < tile_end) {
    ld.load(kg, vg, kv_stride, tile_begin * kTile, p.seqlen, tid);
    ld.store(k_lds[0], v_lds[0], tid);
  }
  __syncthreads();

  const int krow = perm_rows(n);
  for (int it = tile_begin; it < tile_end; ++it) {
    const int cur = (it - tile_begin) & 1;
    const int t0 = it * kTile;
    const bool more = it + 1 < tile_end;
    if (more) ld.load(kg, vg, kv_stride, t0 + kTile, p.seqlen, tid);
    const bool any = (t0 < hi_max) && (t0 + kTile > lo_min);
    if (any) {
      const bool full = (t0 >= lo_max) && (t0 + kTile <= hi_min);
      const __bf16* ks = k_lds[cur];
      const __bf16* vs = v_lds[cur];
      bf16x8 db[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const bf16x8 a = lds_read_b128(ks, off_dual<D>(kb * 32 + krow, 2 * t + h));
          s = mfma32(a, qf[t], s);
        }
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const bf16x8 a = lds_read_b128(vs, off_b128<D>(kb * 32 + krow, 2 * t + h));
          dp = mfma32(a, gf[t], dp);
        }
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
            if (key < kstart || key >= kend) dsv[r] = 0.f;
          }
        }
        db[2 * kb] = pack_bf16(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        db[2 * kb + 1] = pack_bf16(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const bf16x8 a = tr_fragment_dual<D>(ks, 16 * u, 32 * d, lane);
          acc[d] = mfma32(a, db[u], acc[d]);
        }
    }
    if (more) ld.store(k_lds[cur ^ 1], v_lds[cur ^ 1], tid);
    __syncthreads();
  }

  if (q_ok) {
    __bf16* row = p.dq + ((size_t)b * p.seqlen + my_q) * q_stride + hq * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[d][4 * g + e] * p.scale);
        *reinterpret_cast<bf16x4*>(row + 32 * d + 8 * g + 4 * h) = w;
      }
  }
}

template <int D, int NWK, int NWQ, bool CAUSAL>
hipError_t launch_bwd(const BwdParams& p, unsigned phases, hipStream_t stream) {
  if (phases & kBwdDelta) {
    constexpr int RPB = 256 / (D / 8);
    const long nrows = (long)p.batch * p.seqlen * p.hq;
    dim3 grid((unsigned)((nrows + RPB - 1) / RPB));
    hipLaunchKernelGGL((attn_bwd_delta_kernel<D>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDkDv) {
    BwdParams q = p;
    q.num_blk = (p.seqlen + 32 * NWK - 1) / (32 * NWK);
    dim3 grid(p.batch * p.hkv, q.num_blk);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NWK, CAUSAL>), grid, dim3(NWK * 64), 0, stream, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDq) {
    BwdParams q = p;
    q.num_blk = (p.seqlen + 32 * NWQ - 1) / (32 * NWQ);
    dim3 grid(p.batch * p.hq, q.num_blk);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NWQ, CAUSAL>), grid, dim3(NWQ * 64), 0, stream, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t run_bwd(const BwdParams& p, unsigned phases, hipStream_t stream) {
  if (p.head_dim == 128) {
    return p.causal ? launch_bwd<128, 4, 4, true>(p, phases, stream)
                    : launch_bwd<128, 4, 4, false>(p, phases, stream);
  }
  return p.causal ? launch_bwd<64, 4, 4, true>(p, phases, stream) : launch_bwd<64, 4, 4, false>(p, phases, stream);
}

}  // namespace mi355attn
