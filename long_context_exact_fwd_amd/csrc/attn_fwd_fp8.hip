// FP8 (OCP E4M3FN) forward kernel for gfx950.
//
// Same tiled online-softmax method as the bf16 forward ("ms-swift集成FlashAttention
// 2/3，长文本训练更高效", section "FlashAttention 如何破局"), with the FP8 datatype
// that the same page's FA-3 paragraph names and per-tensor scaling of E4M3 data
// as in the Q-Galore section of "ms-swift支持GPU显存碎片整理提升利用率":
//   S = (Q8 K8^T) * descale_q * descale_k * scale, online softmax in fp32,
//   P rounded to E4M3 for the PV product, O = (P8 V8) * descale_v / l,
//   l summed from the fp32 probabilities.
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit
// block scales, fp32 accumulate). Work split as in the bf16 kernel: waves of
// 32 queries, 4 per workgroup with two workgroups per CU, or 8 per workgroup
// with one per CU (fwd_fp8_block_waves()), 64-key K/V tiles copied into LDS
// by buffer loads, double-buffered.
//   * S^T = K Q^T: lane (n, h) supplies bytes [64t + 32h, +32) of its row for
//     both operands (the lane-to-k order of an MFMA is the same for A and B,
//     so any common byte choice contracts every d exactly once).
//   * P^T as the B operand of O^T += V^T P^T: byte 8q + e of lane (n, h) is the
//     probability of key 16q + 8h + e, which is where the score C layout of
//     the perm_rows key order already puts it (register 8(q & 1) + e of key
//     block q / 2).
//   * V^T fragments come from ds_read_b64_tr_b8: in each 16-lane group,
//     destination lane t gets byte t % 8 of the 8-byte segments addressed by
//     source lanes t / 8 + 2e (e = 0..7), so source lane s points at key row
//     16q + 8h + s / 2, column half s % 2 of the lane group's 16 d-columns.
//   * v_cvt_pk_fp8_f32 rounds to nearest even and turns values above 464
//     into NaN. P = 2^(S c - m + 8): the offset of 8 keeps small
//     probabilities in E4M3's normal range instead of flushing them to zero,
//     and cancels in O = acc / l (it is added back in the LSE).
//   * Running maximum m: as in the bf16 forward, a row keeps the maximum of
//     its first tile, here raised by kP8Margin = 6, so P stays below 448
//     while later scores exceed that tile's maximum by less than about 6.8
//     (log2 units): no tile maximum and no rescale in the loop, 6-16 %
//     faster on MI355X, the kernel being bound by its VALU work. A
//     probability beyond the range becomes NaN and reaches O's accumulator;
//     a wave that finds one redoes its rows with the tracked maximum, moved
//     when a tile's maximum exceeds it by 0.5, which keeps P at most 2^8.5.
#define ATTN_LDS_FAULT_WORD g_lds_fault_fp8
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;       // head dim (bytes per fp8 row)
constexpr int kBN = 64;       // keys per tile
constexpr int kTileBytes = kBN * kD;
constexpr float kP8Offset = 8.0f;       // log2 units subtracted from the running maximum
constexpr float kP8Threshold = 0.5f;    // lazy rescale threshold for the fp8 path
constexpr float kP8Margin = 6.0f;       // first-tile maximum raised by this (log2 units) in the fast pass

// 16 bytes of a K tile, and the transposing 8-byte read of a V tile.
__device__ __forceinline__ u32x4 lds_read_u8x16(const uint8_t* p) {
  ATTN_LDS_CHECK(p, 16u, 1u, return u32x4{});
  return *LDS_PTR(const u32x4, p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  ATTN_LDS_CHECK(p, 8u, 1u, return i32x2{});
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, const_cast<uint8_t*>(p)));
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats 0/0 = E4M3 for A and B; E8M0 block scales 127 = 1.0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// MERGE: the epilogue folds the result into the running (o_acc, lse_acc) of a
// ring step instead of writing o and lse.
template <bool CAUSAL, int WAVES, bool MERGE>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void attn_fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int kWaves = WAVES;
  constexpr int kBM = 32 * kWaves;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[kTileBytes];
  __shared__ int red[2][kWaves];
  constexpr int NI = kTileBytes / (kWaves * 1024);  // DMA instructions per wave per tensor and tile

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int hq = bh - b * p.hq;
  const int hk = hq / (p.hq / p.hkv);
  // blockIdx.y = rank * key_split + share, ranks from the heaviest block down
  const int ks = p.key_split;
  const int yrank = (int)blockIdx.y / ks;
  const int share = (int)blockIdx.y - yrank * ks;
  const int qblk = p.num_qblk - 1 - yrank;
  const int my_q = qblk * kBM + wave * 32 + n;
  const bool q_ok = my_q < p.seqlen;

  const int q_stride = p.hq * kD;  // bytes
  const int kv_stride = p.hkv * kD;
  const uint8_t* qg = p.q + (size_t)b * p.seqlen * q_stride + hq * kD;
  const uint8_t* kg = p.k + (size_t)b * p.seqlen * kv_stride + hk * kD;
  const uint8_t* vg = p.v + (size_t)b * p.seqlen * kv_stride + hk * kD;

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

  // Q as B operands: k-step t, bytes [64t + 32h, +32) of the lane's query row.
  i32x8 qf[2];
  {
    const uint8_t* qrow = qg + (size_t)min(my_q, p.seqlen - 1) * q_stride + 32 * h;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * t);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * t + 16);
      qf[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  // LDS byte offsets (tile-relative).
  int koff[2][2];  // [t][half of the 32 bytes]: K row perm_rows(n), chunk 4t + 2h + i
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) koff[t][i] = fp8_k_frag(lane, t, i);
  int voff[4];  // V^T source address of key step q = 0 for d block db
#pragma unroll
  for (int db = 0; db < 4; ++db) voff[db] = fp8_v_frag(lane, db);
  uint32_t ld_koff[NI], ld_voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int off = fp8_dma_byte(i, kWaves, wave, lane);
    ld_koff[i] = fp8_dma_src_k(off, kv_stride);
    ld_voff[i] = fp8_dma_src_v(off, kv_stride);
  }
  auto issue_tile = [&](int t0, auto buf_c) {
    uint8_t* kd = decltype(buf_c)::value ? k_lds1 : k_lds0;
    uint8_t* vd = decltype(buf_c)::value ? v_lds1 : v_lds0;
    const uint32_t nbytes = (uint32_t)(p.seqlen - t0) * (uint32_t)kv_stride;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)t0 * kv_stride, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)t0 * kv_stride, nbytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int el = fp8_dma_byte(i, kWaves, wave, 0);
      dma16_buf(rk, ld_koff[i], kd + el);
      dma16_buf(rv, ld_voff[i], vd + el);
    }
  };

  const float dq = p.descale_q[0], dk = p.descale_k[0], dv = p.descale_v[0];
  const float c = p.scale * dq * dk * kLog2e;  // raw fp8 dot product -> log2 units

  f32x16 acc[4];
  float m_run, l_run;
  // First key tile of this lane's row within this workgroup's share.
  const int kfirst = max(kstart, tile_begin * kBN) / kBN * kBN;

  // One pass over the tiles. FAST: a row's running maximum is its maximum
  // over its first tile plus kP8Margin, kept for the rest of the row (no
  // tile maximum, no rescale); a probability that then exceeds the E4M3
  // range turns into NaN in the conversion, and the wave redoes its rows
  // with the tracked maximum (!FAST). A wave that is not `active` only
  // copies tiles and meets the barriers.
  auto run_tiles = [&](auto fast_c, bool active) {
    constexpr bool FAST = decltype(fast_c)::value;
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
      m_run = kMaxInit;
      l_run = 0.f;
    }
    if (tile_begin < tile_end) issue_tile(tile_begin * kBN, std::integral_constant<int, 0>{});
    wait_dma();
    __syncthreads();

  auto tile_body = [&](int it, auto cur_c) {
      constexpr int cur = decltype(cur_c)::value;
      const int t0 = it * kBN;
      if (it + 1 < tile_end) issue_tile(t0 + kBN, std::integral_constant<int, cur ^ 1>{});
      if (active && (t0 < hi_max) && (t0 + kBN > lo_min)) {
        const bool full = (t0 >= lo_max) && (t0 + kBN <= hi_min);
        const uint8_t* ks = cur ? k_lds1 : k_lds0;
        const uint8_t* vs = cur ? v_lds1 : v_lds0;
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = f32x16{};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 lo = lds_read_u8x16(ks + koff[t][0] + kb * 32 * kD);
            const u32x4 hi = lds_read_u8x16(ks + koff[t][1] + kb * 32 * kD);
            const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            s[kb] = mfma_fp8(a, qf[t], s[kb]);
          }
        }
        if (!full) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t0 + kb * 32 + c_key(r, h);
              s[kb][r] = (key < kstart || key >= kend) ? -INFINITY : s[kb][r];
            }
        }
        if (!FAST || __any(t0 == kfirst)) {
          float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = max3f(mx, s[0][r], s[1][r]);
          mx = max_lane_halves(mx);
          const float m_tile = mx * c;
          if (FAST) {
            // rows entering their first tile; a row without keys here keeps kMaxInit
            if (t0 == kfirst && m_tile > kMaxInit) m_run = m_tile + kP8Margin;
          } else if (__any(m_tile > m_run + kP8Threshold)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= alpha;
            m_run = m_new;
          }
        }
        const float neg_m = kP8Offset - m_run;
        // P^T bytes: byte 8q + e = key 16q + 8h + e = register 8(q & 1) + e of key block q / 2
        i32x8 pf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float e[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            e[r] = fast_exp2(__builtin_fmaf(s[kb][r], c, neg_m));
            l_run += e[r];
          }
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w], e[4 * w + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w + 2], e[4 * w + 3], word, true);
            pf[4 * kb + w] = word;
          }
        }
        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          i32x8 a;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const i32x2 t = lds_read_tr8(vs + voff[db] + q * 16 * kD);
            a[2 * q] = t[0];
            a[2 * q + 1] = t[1];
          }
          acc[db] = mfma_fp8(a, pf, acc[db]);
        }
      }
      wait_dma();
      __syncthreads();
    };


    for (int it = tile_begin; it < tile_end; it += 2) {
      tile_body(it, std::integral_constant<int, 0>{});
      if (it + 1 < tile_end) tile_body(it + 1, std::integral_constant<int, 1>{});
    }
  };

  run_tiles(std::true_type{}, true);
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) nan = nan || (acc[i][r] != acc[i][r]);
  const bool redo = __any(nan);
  if (__syncthreads_or(redo)) run_tiles(std::false_type{}, redo);

  // O = acc * descale_v / l; LSE = (m - offset + log2 l) * ln 2
  const float l_tot = sum_lane_halves(l_run);
  const float inv = l_tot > 0.f ? dv / l_tot : 0.f;
  if (q_ok && ks > 1) {
    // key split: this share's O (fp32, descaled) and m - offset + log2 l
    const size_t plane = (size_t)p.batch * p.seqlen * p.hq * kD;
    float* orow = p.part_o + (size_t)share * plane + ((size_t)b * p.seqlen + my_q) * (size_t)(p.hq * kD) + hq * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (h == 0) {
      p.part_lse[(((size_t)share * p.batch + b) * p.hq + hq) * p.seqlen + my_q] =
          l_tot > 0.f ? m_run - kP8Offset + __log2f(l_tot) : -INFINITY;
    }
  } else if (MERGE) {
    // With L_a = LSE_acc log2 e and this call's L_p = m - offset + log2 l,
    // M = max(L_a, L_p), T = 2^(L_a - M) + 2^(L_p - M):
    //   O = (2^(L_a - M) / T) O_acc + (2^(m - offset - M) d_v / T) acc,
    //   LSE = (M + log2 T) ln 2;
    // both lanes of a row read LSE_acc before the h = 0 lane stores it.
    if (q_ok && l_tot > 0.f) {
      const size_t ri = ((size_t)b * p.seqlen + my_q) * (size_t)(p.hq * kD) + hq * kD;
      const size_t li = ((size_t)b * p.hq + hq) * p.seqlen + my_q;
      const float la = p.accumulate ? p.lse_acc[li] * kLog2e : -INFINITY;
      const float lp = m_run - kP8Offset + __log2f(l_tot);
      const float mm = fmaxf(la, lp);
      const float wa = fast_exp2(la - mm);
      const float tot = wa + fast_exp2(lp - mm);
      const float rt = 1.0f / tot;
      const float ca = wa * rt, cp = fast_exp2(m_run - kP8Offset - mm) * dv * rt;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* dst = reinterpret_cast<f32x4*>(p.o_acc + ri + 32 * db + 8 * g + 4 * h);
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
    __bf16* orow = p.o + ((size_t)b * p.seqlen + my_q) * (size_t)(p.hq * kD) + hq * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
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
          l_tot > 0.f ? (m_run - kP8Offset + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <bool CAUSAL>
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  Fp8FwdParams q = p;
  if (q.key_split < 1 || q.part_o == nullptr || q.part_lse == nullptr) q.key_split = 1;
  const int waves = q.key_split > 1 ? 4 : fwd_fp8_block_waves(q.seqlen, q.causal, q.cu_seqlens != nullptr);
  q.num_qblk = (p.seqlen + 32 * waves - 1) / (32 * waves);
  dim3 grid(p.batch * p.hq, q.num_qblk * q.key_split);
  // with a key split the kernel writes only partials, which the combine merges
  const bool merge = q.o_acc != nullptr && q.key_split == 1;
  if (waves == 8) {
    if (merge) {
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, 8, true>), grid, dim3(8 * 64), 0, stream, q);
    } else {
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, 8, false>), grid, dim3(8 * 64), 0, stream, q);
    }
  } else {
    if (merge) {
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, 4, true>), grid, dim3(4 * 64), 0, stream, q);
    } else {
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, 4, false>), grid, dim3(4 * 64), 0, stream, q);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || q.key_split == 1) return e;
  FwdParams c{};
  c.o = q.o;
  c.lse = q.lse;
  c.part_o = q.part_o;
  c.part_lse = q.part_lse;
  c.batch = q.batch;
  c.seqlen = q.seqlen;
  c.hq = q.hq;
  c.head_dim = kD;
  c.key_split = q.key_split;
  c.o_acc = q.o_acc;  // ring merge: the combine merges every row (the fp8 path has no few-key kernel)
  c.lse_acc = q.lse_acc;
  c.o_out = q.o_out;
  c.accumulate = q.accumulate;
  c.few_rows_apart = 0;
  return run_fwd_combine(c, stream);
}

}  // namespace

hipError_t run_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  return p.causal ? launch_fwd_fp8<true>(p, stream) : launch_fwd_fp8<false>(p, stream);
}

#ifdef ATTN_DEBUG
hipError_t lds_faults_fp8(unsigned int* out) { return take_lds_fault_word(out); }
#endif

}  // namespace mi355attn
