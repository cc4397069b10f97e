// bf16 forward kernel for gfx950.
//
// The method is the tiled, fused attention of "ms-swift集成FlashAttention 2/3，
// 长文本训练更高效" (section "FlashAttention 如何破局"): a Q block stays on chip,
// K/V blocks stream through on-chip memory, and a running maximum plus
// normaliser per row replace the full softmax, so only O (and the
// log-sum-exp) reach global memory. The FA-2 paragraph of the same page names
// double-buffered loads; here K and V tiles are double-buffered through LDS.
//
// Work split (one workgroup per (b, h_q, block of 32*NW queries)):
//   * each wave owns 32 queries; its Q slice sits in VGPRs as the B operand
//     of S^T = K Q^T (32 keys x 32 queries per MFMA block), so every lane owns
//     one query column and the row statistics need no cross-lane work except
//     one exchange between the two lane halves;
//   * K rows are loaded through perm_rows, which puts the probabilities in
//     exactly the register order the B operand of O^T += V^T P^T needs;
//   * V^T fragments come from the transposing LDS read, so V stays row-major;
//   * 64-key tiles; tiles entirely outside a wave's visible keys are skipped,
//     tiles partly outside are masked per element.
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

constexpr int kBN = 64;  // keys per tile

template <int D, int NW>
struct FwdTileLoader {
  static constexpr int kThreads = NW * 64;
  static constexpr int kChunks = kBN * D / 8;  // 16-byte chunks per tile
  static constexpr int kPer = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile chunks must divide evenly");
  u32x4 k[kPer], v[kPer];

  __device__ __forceinline__ void load(const __bf16* kg, const __bf16* vg, int row_stride, int t0, int seqlen,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int g = t0 + row;
      const bool ok = g < seqlen;
      const size_t off = (size_t)(ok ? g : 0) * row_stride + ch * 8;
      k[i] = load16_pred(kg + off, ok);
      v[i] = load16_pred(vg + off, ok);
    }
  }
  __device__ __forceinline__ void store(__bf16* ks, __bf16* vs, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      lds_store16(ks, off_b128<D>(row, ch), k[i]);
      lds_store16(vs, off_tr<D>(row, ch), v[i]);
    }
  }
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = 32 * NW;
  constexpr int KS = D / 16;  // k-steps of the score product
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kBN * D];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kBN * D];
  __shared__ int red[4][NW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int hq = bh - b * p.hq;
  const int hk = hq / (p.hq / p.hkv);
  const int qblk = p.num_qblk - 1 - (int)blockIdx.y;  // heaviest blocks first
  const int q0 = qblk * BM;
  const int my_q = q0 + wave * 32 + n;
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
  const int tile_begin = wg_hi > wg_lo ? wg_lo / kBN : 0;
  const int tile_end = wg_hi > wg_lo ? (wg_hi + kBN - 1) / kBN : 0;

  // Q slice of this wave as B operands: lane (n, h) holds Q[my_q][16t + 8h .. +7]
  bf16x8 qf[KS];
  {
    const __bf16* qrow = qg + (size_t)(q_ok ? my_q : 0) * q_stride + 8 * h;
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[t] = as_bf16x8(load16_pred(qrow + 16 * t, q_ok));
  }

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = kMaxInit;  // running maximum (scaled, log2 units)
  float l_run = 0.f;       // partial row sum over this lane's keys
  const float c = p.scale_log2e;

  FwdTileLoader<D, NW> ld;
  if (tile_begin < tile_end) {
    ld.load(kg, vg, kv_stride, tile_begin * kBN, p.seqlen, tid);
    ld.store(k_lds[0], v_lds[0], tid);
  }
  __syncthreads();

  const int krow = perm_rows(n);
  for (int it = tile_begin; it < tile_end; ++it) {
    const int cur = (it - tile_begin) & 1;
    const int t0 = it * kBN;
    const bool more = it + 1 < tile_end;
    if (more) ld.load(kg, vg, kv_stride, t0 + kBN, p.seqlen, tid);

    const bool any = (t0 < hi_max) && (t0 + kBN > lo_min);
    if (any) {
      const bool full = (t0 >= lo_max) && (t0 + kBN <= hi_min);
      const __bf16* ks = k_lds[cur];
      const __bf16* vs = v_lds[cur];
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const bf16x8 a = lds_read_b128(ks, off_b128<D>(kb * 32 + krow, 2 * t + h));
          s[kb] = mfma32(a, qf[t], s[kb]);
        }
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t0 + kb * 32 + c_key(r, h);
            if (key < kstart || key >= kend) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = wave_max_halves(mx);
      const float m_tile = mx * c;
      if (__any(m_tile > m_run + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
        m_run = m_new;
      }
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          e[r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_run));
          l_run += e[r];
        }
        pb[2 * kb] = pack_bf16(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        pb[2 * kb + 1] = pack_bf16(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = tr_fragment<D>(vs, 16 * u, 32 * db, lane);
          acc[db] = mfma32(a, pb[u], acc[db]);
        }
    }
    if (more) ld.store(k_lds[cur ^ 1], v_lds[cur ^ 1], tid);
    __syncthreads();
  }

  // epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok) {
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

template <int D, int NW, bool CAUSAL>
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  q.num_qblk = (p.seqlen + 32 * NW - 1) / (32 * NW);
  dim3 grid(p.batch * p.hq, q.num_qblk);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, CAUSAL>), grid, dim3(NW * 64), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

hipError_t run_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  constexpr int NW = 8;
  if (p.head_dim == 128) {
    return p.causal ? launch_fwd<128, NW, true>(p, stream) : launch_fwd<128, NW, false>(p, stream);
  }
  return p.causal ? launch_fwd<64, NW, true>(p, stream) : launch_fwd<64, NW, false>(p, stream);
}

}  // namespace mi355attn
