// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, wave64), checked on gfx950:
//   A (32 x 16): lane l holds row l % 32, k = 8 * (l / 32) + 0..7
//   B (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + 0..7
//   C (32 x 32): lane l holds column l % 32, rows 8 * (r / 4) + 4 * (l / 32) + r % 4, r = 0..15
// The k order inside one product is free as long as A and B agree, which the
// kernels use to permute keys so that a score tile in C layout can feed the
// next product as its B operand without any data movement.
//
// ds_read_b64_tr_b16 (transposing LDS read), checked on gfx950: in each group
// of 16 lanes, source lane 16g + j supplies the address of 4 consecutive
// 16-bit elements; destination lane 16g + t receives element t % 4 of the
// sources 16g + t / 4 + 4e, e = 0..3 (in that order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_index.h"

namespace mi355attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Debug builds (-DATTN_DEBUG, linked into libmi355attn_debug.so) check every
// LDS access made through the helpers below before issuing it: the access
// must lie inside the kernel's static LDS allocation and be aligned to its
// size (lds_access_ok). A failing access is not made (a read returns zeros, a
// store or tile copy is dropped), so no kernel reaches LDS outside its
// allocation, and it sets a bit of this source file's fault word: 1 for a
// read, 2 for a store, 4 for a tile copy. The C ABI then synchronises after
// each call, reads and clears the words and returns ATTN_ERR_DEBUG_CHECK if
// one is set. Device variables belong to one source file here, so each
// kernel file names its word (ATTN_LDS_FAULT_WORD) before including this
// header. Fixed-shape arrays indexed by wave, lane or compile-time slot
// (the reduction scratch, the dK/dV probability exchange) are not routed
// through the checks; their bounds hold by construction. Release builds
// compile none of this.
#ifdef ATTN_DEBUG
#ifndef ATTN_LDS_FAULT_WORD
#error "define ATTN_LDS_FAULT_WORD before including attn_device.h in a debug build"
#endif
__device__ unsigned int ATTN_LDS_FAULT_WORD;
__device__ __forceinline__ bool lds_ok(const void* p, uint32_t bytes, unsigned int bit) {
  const uint32_t addr = (uint32_t)(uintptr_t)LDS_PTR(const char, p);
  const uint32_t align = bytes >= 16u ? 16u : bytes;
  if (mi355attn::lds_access_ok(addr, bytes, align, __builtin_amdgcn_groupstaticsize())) return true;
  atomicOr(&ATTN_LDS_FAULT_WORD, bit);
  return false;
}
#define ATTN_LDS_CHECK(p, bytes, bit, on_fail) \
  if (!lds_ok((p), (bytes), (bit))) on_fail
// Reads and clears this file's fault word on the current device.
static inline hipError_t take_lds_fault_word(unsigned int* out) {
  const unsigned int zero = 0;
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(ATTN_LDS_FAULT_WORD), sizeof(unsigned int));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(ATTN_LDS_FAULT_WORD), &zero, sizeof(unsigned int));
  return e;
}
#else
#define ATTN_LDS_CHECK(p, bytes, bit, on_fail)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A running row maximum below any real scaled score; exp2(-1e30 - x) == 0.
constexpr float kMaxInit = -1.0e30f;
// Where the bf16 forward tracks a running maximum (its redo pass), it is only
// moved when the tile maximum exceeds it by more than this (log2 units). Probabilities are then at most 2^8 before
// normalisation, well inside fp32 and bf16 range; the final division uses
// the same offset, so the result is unchanged.
constexpr float kRescaleThreshold = 8.0f;
// The bf16 forward's first-tile maximum is kept while each lane's
// probability sum over a tile stays at most this (2^64): P, the row sum and
// O's accumulator then stay far inside the fp32 and bf16 range.
constexpr float kTileSumLimit = 18446744073709551616.0f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_halves(float x) {
  // lanes l and l ^ 32 hold the same query column
  return fmaxf(x, __shfl_xor(x, 32));
}

// v_permlane32_swap exchanges the upper half of one copy of x with the lower
// half of another, so the two results hold, lane by lane, x[l] and x[l ^ 32]
// (in one order or the other). A commutative combination of the two is the
// same in every lane of a pair, whichever way round the halves come back.
__device__ __forceinline__ float max_lane_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* base, int elem_off) {
  ATTN_LDS_CHECK(base + elem_off, 16u, 1u, return bf16x8{});
  return *LDS_PTR(const bf16x8, base + elem_off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* base, int elem_off) {
  ATTN_LDS_CHECK(base + elem_off, 8u, 1u, return bf16x4{});
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, const_cast<__bf16*>(base) + elem_off));
}

// Plain 16-byte LDS loads and stores through a generic pointer into a
// __shared__ array (fp32 row statistics, the few-key kernel's rows).
template <typename T>
__device__ __forceinline__ T lds_load16(const void* p) {
  static_assert(sizeof(T) == 16, "16-byte accesses only");
  ATTN_LDS_CHECK(p, 16u, 1u, return T{});
  return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_store16g(void* p, const T& v) {
  static_assert(sizeof(T) == 16, "16-byte accesses only");
  ATTN_LDS_CHECK(p, 16u, 2u, return);
  *reinterpret_cast<T*>(p) = v;
}

// Two transposing reads, 4 rows apart in a TR tile: elem_off is the first
// read's offset and row_delta the element distance of the second.
__device__ __forceinline__ bf16x8 tr_read_pair(const __bf16* tile, int elem_off, int row_delta) {
  const bf16x4 lo = lds_read_tr(tile, elem_off);
  const bf16x4 hi = lds_read_tr(tile, elem_off + row_delta);
  bf16x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

// Direct global -> LDS copy (global_load_lds_dwordx4): lane L of the wave
// copies 16 bytes from g into lds_wave_base + 16 L. lds_wave_base must be the
// same for every lane of the wave (it goes to M0). Completion is tracked by
// vmcnt, so wait_dma() must precede the barrier after which the data is read.
__device__ __forceinline__ void dma16(const void* g, const void* lds_wave_base) {
  ATTN_LDS_CHECK(static_cast<const char*>(lds_wave_base) + 16 * __lane_id(), 16u, 4u, return);
  __builtin_amdgcn_global_load_lds(g, LDS_PTR(void, const_cast<void*>(lds_wave_base)), 16, 0, 0);
}
// Buffer resource over [base, base + nbytes) (raw, stride 0): a load whose
// per-lane offset is past nbytes returns zeros, which handles ragged tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
// buffer_load_dwordx4 ... lds: lane L copies 16 bytes at byte offset voff of
// the buffer into lds_wave_base + 16 L (same M0 rule as dma16).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, const void* lds_wave_base) {
  ATTN_LDS_CHECK(static_cast<const char*>(lds_wave_base) + 16 * __lane_id(), 16u, 4u, return);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, const_cast<void*>(lds_wave_base)), 16, voff, 0, 0, 0);
}
// s_waitcnt vmcnt(0), other counters left alone (expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Two transposing reads at independent offsets (dual tiles: the swizzle of
// row r + 4 differs from that of row r).
__device__ __forceinline__ bf16x8 tr_read2(const __bf16* tile, int off_lo, int off_hi) {
  const bf16x4 lo = lds_read_tr(tile, off_lo);
  const bf16x4 hi = lds_read_tr(tile, off_hi);
  bf16x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

__device__ __forceinline__ u32x4 load16(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_pred(const __bf16* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}
__device__ __forceinline__ void lds_store16(__bf16* base, int elem_off, u32x4 v) {
  ATTN_LDS_CHECK(base + elem_off, 16u, 2u, return);
  *LDS_PTR(u32x4, base + elem_off) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight fp32 values -> bf16x8, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16(float a0, float a1, float a2, float a3, float a4, float a5,
                                            float a6, float a7) {
  bf16x8 o;
  o[0] = (__bf16)a0; o[1] = (__bf16)a1; o[2] = (__bf16)a2; o[3] = (__bf16)a3;
  o[4] = (__bf16)a4; o[5] = (__bf16)a5; o[6] = (__bf16)a6; o[7] = (__bf16)a7;
  return o;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

}  // namespace mi355attn
