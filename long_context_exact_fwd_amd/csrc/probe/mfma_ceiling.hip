// Matrix-pipe ceiling probe for gfx950 (measurement only, not part of the
// attention library): the rate at which this GPU sustains
// v_mfma_f32_32x32x16_bf16 when nothing else limits it, and the shader clock
// it runs at meanwhile. The attention kernels' roofline fractions are quoted
// against the 2.5 PF/s datasheet peak; this figure says how much of that the
// chip delivers under a pure MFMA load.
//
// The MFMA's power, and with it the clock the power limit allows, depends on
// the operand bits. Two operand patterns:
//   RANDOM: eight A and eight B fragments per lane with random signs,
//     exponents 2^-1..2^1 and random mantissas (the spread of N(0, 1) data),
//     rotated so that every MFMA sees different inputs than the one before;
//   otherwise: one A and one B fragment of small multiples of 2^-7 (few set
//     bits, no change between MFMAs).
// One workgroup of 8 waves per CU (two waves per SIMD, the attention kernels'
// occupancy). Every wave runs `iters` rounds of 8 independent accumulation
// chains on register operands: no memory traffic inside the loop. Lane 0 of
// wave 0 records the shader-clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around the loop; their ratio gives the
// clock. Results go out through ordinary vector stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;
constexpr int kWavesPerGroup = 8;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // integer finaliser (xor-shift / multiply rounds), any fixed bijection will do
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 with a random sign, exponent 126..128 and random 7-bit mantissa
__device__ __forceinline__ __bf16 random_bf16(uint32_t key) {
  const uint32_t r = mix32(key);
  const uint32_t bits = ((r & 1u) << 15) | ((126u + (r >> 1) % 3u) << 7) | ((r >> 8) & 0x7fu);
  return __builtin_bit_cast(__bf16, (uint16_t)bits);
}

template <bool RANDOM>
__global__ __launch_bounds__(kWavesPerGroup * 64, 1) void mfma_ceiling_kernel(float* out, uint64_t* clocks,
                                                                               int iters) {
  const int tid = threadIdx.x;
  const uint32_t gid = blockIdx.x * blockDim.x + tid;
  constexpr int NF = RANDOM ? kChains : 1;
  bf16x8 a[NF], b[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (RANDOM) {
        a[f][e] = random_bf16(gid * 128u + f * 16u + e);
        b[f][e] = random_bf16(gid * 128u + f * 16u + 8u + e);
      } else {
        a[f][e] = (__bf16)((float)((tid + e) & 7) * 0.0078125f);
        b[f][e] = (__bf16)((float)((tid * 3 + e) & 7) * 0.0078125f);
      }
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % NF], b[(c + 3) % NF], acc[c], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[gid] = s;
  if (tid == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Flops one launch performs: groups * 8 waves * iters * 8 chains * 2*32*32*16.
double mfma_ceiling_flops(int groups, int iters) {
  return (double)groups * kWavesPerGroup * iters * kChains * (2.0 * 32 * 32 * 16);
}

// Enqueues the probe on `stream`. random_operands: 1 for the N(0, 1)-like
// rotating operands, 0 for the constant low-entropy ones. out: groups * 512
// floats; clocks: 2 * groups uint64 (shader-clock ticks, 100 MHz ticks of
// wave 0 of each workgroup). Returns the hipError_t of the launch (0 on
// success), or -1 for bad arguments.
int mfma_ceiling_launch(float* out, uint64_t* clocks, int groups, int iters, int random_operands, void* stream) {
  if (out == nullptr || clocks == nullptr || groups < 1 || iters < 1) return -1;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (random_operands) {
    hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3(groups), dim3(kWavesPerGroup * 64), 0, s, out, clocks, iters);
  } else {
    hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3(groups), dim3(kWavesPerGroup * 64), 0, s, out, clocks,
                       iters);
  }
  return (int)hipGetLastError();
}

}  // extern "C"
