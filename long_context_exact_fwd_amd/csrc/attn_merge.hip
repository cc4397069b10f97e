// Merge of a partial attention result into a running one (Ring-Attention step).
//
// Ring-Attention passes K/V blocks around a ring of devices, and each device
// accumulates partial attention results until it has seen the whole context
// (FlashAttention page "ms-swift集成FlashAttention 2/3，长文本训练更高效",
// sequence-parallel section, Ring-Attention paragraph). Attention of a query
// row over two disjoint key sets A and B combines exactly into attention over
// A ∪ B: the softmax denominators add, so with M = max(LSE_A, LSE_B)
//   w_A = e^(LSE_A - M), w_B = e^(LSE_B - M),
//   O = (w_A O_A + w_B O_B) / (w_A + w_B),  LSE = M + ln(w_A + w_B).
// A part with no visible key has LSE = -inf and weight 0; if neither has
// one, O = 0 and LSE = -inf.
//
// Memory-bound: each thread handles 8 consecutive d of one (b, s, h) row,
// reading 16 bytes of the bf16 part and 32 of the fp32 accumulator with
// vector loads, so a wave reads whole rows contiguously. The D / 8 threads of
// a row sit in one wave; the one holding d = 0..7 writes the row's LSE after
// every lane of the wave has read it.
#define ATTN_LDS_FAULT_WORD g_lds_fault_merge
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {

namespace {

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 8;  // threads per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long nrows = (long)p.batch * p.seqlen * p.heads;
  const long row = t / TPR;  // (b, s, h) in [B, S, H] order
  if (row >= nrows) return;
  const int sub = (int)(t - row * TPR);
  const int h = (int)(row % p.heads);
  const long bs = row / p.heads;
  const int s = (int)(bs % p.seqlen);
  const long b = bs / p.seqlen;
  const long li = (b * p.heads + h) * p.seqlen + s;  // LSE index in [B, H, S]
  const size_t off = (size_t)row * D + sub * 8;

  const float l2 = p.lse_part[li];
  const float l1 = p.accumulate ? p.lse_acc[li] : -INFINITY;
  const bf16x8 op = as_bf16x8(load16(p.o_part + off));
  f32x4 o1a = f32x4{}, o1b = f32x4{};
  if (p.accumulate) {
    o1a = *reinterpret_cast<const f32x4*>(p.o_acc + off);
    o1b = *reinterpret_cast<const f32x4*>(p.o_acc + off + 4);
  }
  const float m = fmaxf(l1, l2);
  float a1 = 0.f, a2 = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float w1 = fast_exp2((l1 - m) * kLog2e);  // exp2(-inf) = 0
    const float w2 = fast_exp2((l2 - m) * kLog2e);
    const float tot = w1 + w2;                       // >= 1: the larger weight is 1
    const float inv = 1.0f / tot;
    a1 = w1 * inv;
    a2 = w2 * inv;
    lse = m + __log2f(tot) * kLn2;
  }
  f32x4 ra, rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = a1 * o1a[e] + a2 * (float)op[e];
    rb[e] = a1 * o1b[e] + a2 * (float)op[4 + e];
  }
  *reinterpret_cast<f32x4*>(p.o_acc + off) = ra;
  *reinterpret_cast<f32x4*>(p.o_acc + off + 4) = rb;
  if (p.o_out != nullptr) {
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = (__bf16)ra[e];
      w[4 + e] = (__bf16)rb[e];
    }
    *reinterpret_cast<bf16x8*>(p.o_out + off) = w;
  }
  if (sub == 0) p.lse_acc[li] = lse;
}

}  // namespace

hipError_t run_merge(const MergeParams& p, hipStream_t stream) {
  const long nthreads = (long)p.batch * p.seqlen * p.heads * (p.head_dim / 8);
  const dim3 grid((unsigned)((nthreads + 255) / 256));
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

#ifdef ATTN_DEBUG
hipError_t lds_faults_merge(unsigned int* out) { return take_lds_fault_word(out); }
#endif

}  // namespace mi355attn
