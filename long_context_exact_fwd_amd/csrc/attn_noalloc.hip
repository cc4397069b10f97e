// attn_bwd_noalloc: the backward for callers that cannot allocate device
// memory (code under HIP graph capture, allocation-free serving loops). Its
// workspace (Delta, LSE*log2e, the work order and the split partials) lives in
// a fixed array inside the library instead of a caller buffer.
//
// `scratch` below is a device variable: in host code its name is only a
// stand-in, so every host use goes through the address that
// hipGetSymbolAddress returns for the current device. Each device holds its
// own copy (at its own address), taken once per device on the first call
// there and kept for the life of the process.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
__device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device; null until looked up

// Device address of `scratch` on the calling thread's current device.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int batch, int hq, int hkv, int seqlen,
                             int head_dim, int causal, const int32_t* cu_seqlens, int num_seqs, float scale,
                             attn_stream_t stream) {
  attn_status st = mi355attn::bwd_check(ATTN_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, nullptr, false, batch, hq,
                                        hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  // The splits attn_bwd would choose when their partials fit; otherwise none
  // (the same kernels, summing a GQA group's heads and a block's key tiles in
  // one workgroup); otherwise the request is too large for the scratch.
  int hs = mi355attn::bwd_head_split(batch, hq, hkv, seqlen);
  int ks = mi355attn::bwd_key_split(batch, hq, seqlen);
  if (mi355attn::bwd_workspace_size(batch, hq, hkv, seqlen, head_dim, hs, ks) > ATTN_NOALLOC_SCRATCH_BYTES) {
    hs = 1;
    ks = 1;
    if (mi355attn::bwd_workspace_size(batch, hq, hkv, seqlen, head_dim, 1, 1) > ATTN_NOALLOC_SCRATCH_BYTES)
      return ATTN_ERR_SCRATCH_TOO_SMALL;
  }
  void* ws = nullptr;
  st = mi355attn::hip_result(scratch_on_current_device(&ws));
  if (st != ATTN_OK) return st;
  return mi355attn::bwd_launch(ATTN_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, ws, hs, ks, batch, hq, hkv, seqlen,
                               head_dim, causal, cu_seqlens, num_seqs, scale, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
