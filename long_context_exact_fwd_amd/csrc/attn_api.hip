// C ABI of libmi355attn.so: argument checks, then kernel launches on the
// caller's stream. Every check runs before any HIP call (the optional
// ATTN_VALIDATE copy of cu_seqlens runs after them and before any launch).
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element count of any tensor must fit the kernels' 32-bit row
// arithmetic per (batch) slice and 64-bit offsets overall.
attn_status check_common(int batch, int hq, int hkv, int seqlen, int head_dim, int causal,
                         const int32_t* cu_seqlens, int num_seqs, float scale) {
  if (batch < 1 || hq < 1 || hkv < 1 || seqlen < 1 || head_dim < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (hq % hkv != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (cu_seqlens != nullptr) {
    if (batch != 1 || num_seqs < 1 || num_seqs > seqlen) return ATTN_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return ATTN_ERR_INVALID_ARGUMENT;
  } else if (num_seqs != 0) {
    return ATTN_ERR_INVALID_ARGUMENT;
  }
  // per-(b) slice of Q must be addressable with 32-bit row offsets times D
  if ((long long)seqlen * hq * head_dim > (long long)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// ATTN_VALIDATE=1: copy cu_seqlens to the host (synchronising `stream`) and
// check that it is a valid prefix-sum array before anything is launched.
attn_status validate_cu(const int32_t* cu, int num_seqs, int seqlen, hipStream_t stream) {
  const char* env = getenv("ATTN_VALIDATE");
  if (cu == nullptr || env == nullptr || strcmp(env, "1") != 0) return ATTN_OK;
  std::vector<int32_t> h((size_t)num_seqs + 1);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
  }
  if (h[0] != 0 || h[num_seqs] != seqlen) return ATTN_ERR_INVALID_ARGUMENT;
  for (int s = 0; s < num_seqs; ++s)
    if (h[s + 1] <= h[s]) return ATTN_ERR_INVALID_ARGUMENT;
  return ATTN_OK;
}

}  // namespace

namespace mi355attn {

int fwd_block_waves_env() {
  const char* env = getenv("ATTN_FWD_WAVES");
  if (env == nullptr) return 0;
  return atoi(env);
}

int bwd_dq_waves_env() {
  const char* env = getenv("ATTN_DQ_WAVES");
  if (env == nullptr) return 0;
  return atoi(env);
}

attn_status hip_result(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status launched(hipError_t e, hipStream_t stream) {
  const attn_status st = hip_result(e);
#ifdef ATTN_DEBUG
  if (st != ATTN_OK) return st;
  hipError_t r = hipStreamSynchronize(stream);
  unsigned int faults = 0;
  for (hipError_t (*take)(unsigned int*) : {lds_faults_fwd, lds_faults_fp8, lds_faults_bwd, lds_faults_merge}) {
    unsigned int w = 0;
    if (r == hipSuccess) r = take(&w);
    faults |= w;
  }
  if (r != hipSuccess) return hip_result(r);
  if (faults != 0) return ATTN_ERR_DEBUG_CHECK;
#else
  (void)stream;
#endif
  return st;
}

attn_status bwd_check(unsigned phases, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, const void* workspace, bool need_workspace,
                      int batch, int hq, int hkv, int seqlen, int head_dim, int causal, const int32_t* cu_seqlens,
                      int num_seqs, float scale) {
  if (phases == 0u || (phases & ~7u) != 0u) return ATTN_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARGUMENT;
  if (need_workspace && (!workspace || !aligned16(workspace))) return ATTN_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status st = check_common(batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status bwd_launch(unsigned phases, const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* workspace, int head_split, int key_split,
                       int batch, int hq, int hkv, int seqlen, int head_dim, int causal, const int32_t* cu_seqlens,
                       int num_seqs, float scale, hipStream_t stream, const float* descale_q, const float* descale_k,
                       const float* descale_v, int accumulate) {
  const attn_status st = validate_cu(cu_seqlens, num_seqs, seqlen, stream);
  if (st != ATTN_OK) return st;
  BwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<const __bf16*>(o);
  p.lse = lse;
  p.dout = static_cast<const __bf16*>(dout);
  if (accumulate >= 0) {
    p.dq_acc = static_cast<float*>(dq);
    p.dk_acc = static_cast<float*>(dk);
    p.dv_acc = static_cast<float*>(dv);
    p.accumulate = accumulate;
  } else {
    p.dq = static_cast<__bf16*>(dq);
    p.dk = static_cast<__bf16*>(dk);
    p.dv = static_cast<__bf16*>(dv);
  }
  p.stat_stride = stat_stride_for(seqlen);
  char* ws = static_cast<char*>(workspace);
  p.delta = reinterpret_cast<float*>(ws);
  p.lse2 = p.delta + (size_t)batch * hq * p.stat_stride;
  p.order = reinterpret_cast<int*>(ws + bwd_order_offset(batch, hq, seqlen));
  p.head_split = head_split;
  p.key_split = key_split;
  p.dq_waves = bwd_dq_block_waves(seqlen, head_dim, causal, cu_seqlens != nullptr, key_split);
  p.part = head_split > 1 ? reinterpret_cast<float*>(ws + bwd_part_offset(batch, hq, seqlen, head_split, key_split))
                          : nullptr;
  p.dq_part = key_split > 1 ? reinterpret_cast<float*>(ws + bwd_dq_part_offset(batch, hq, hkv, seqlen, head_dim,
                                                                               head_split, key_split))
                            : nullptr;
  p.cu_seqlens = cu_seqlens;
  p.num_seqs = num_seqs;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.seqlen = seqlen;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.descale_v = descale_v;
  return launched(run_bwd(p, phases, stream), stream);
}

}  // namespace mi355attn

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARGUMENT: return "ATTN_ERR_INVALID_ARGUMENT";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    case ATTN_ERR_SCRATCH_TOO_SMALL: return "ATTN_ERR_SCRATCH_TOO_SMALL";
    case ATTN_ERR_DEBUG_CHECK: return "ATTN_ERR_DEBUG_CHECK";
  }
  return "ATTN_ERR_UNKNOWN";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

size_t attn_bwd_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || seqlen <= 0 || head_dim <= 0 || hq % hkv != 0) return 0;
  if ((long long)seqlen * hq * head_dim > (long long)INT32_MAX) return 0;
  return mi355attn::bwd_workspace_size(batch, hq, hkv, seqlen, head_dim);
}

size_t attn_fwd_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || seqlen <= 0 || head_dim <= 0 || hq % hkv != 0) return 0;
  if ((long long)seqlen * hq * head_dim > (long long)INT32_MAX) return 0;
  return mi355attn::fwd_workspace_size(batch, hq, seqlen, head_dim);
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace, int batch,
                     int hq, int hkv, int seqlen, int head_dim, int causal, const int32_t* cu_seqlens, int num_seqs,
                     float scale, attn_stream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace && !aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_common(batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  st = validate_cu(cu_seqlens, num_seqs, seqlen, reinterpret_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  mi355attn::FwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.num_seqs = num_seqs;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.seqlen = seqlen;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.key_split = 1;
  const int ks = mi355attn::fwd_key_split(batch, hq, seqlen);
  if (workspace != nullptr && ks > 1) {
    p.key_split = ks;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          mi355attn::fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks));
  }
  return mi355attn::launched(mi355attn::run_fwd_bf16(p, reinterpret_cast<hipStream_t>(stream)),
                               reinterpret_cast<hipStream_t>(stream));
}

attn_status attn_fwd_merge(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc, void* o_out,
                           int accumulate, void* workspace, int batch, int hq, int hkv, int seqlen, int head_dim,
                           int causal, const int32_t* cu_seqlens, int num_seqs, float scale, attn_stream_t stream) {
  if (!q || !k || !v || !o_acc || !lse_acc) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_acc) || (o_out && !aligned16(o_out)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(lse_acc) & 3u) return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace && !aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
  if (accumulate != 0 && accumulate != 1) return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_common(batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  st = validate_cu(cu_seqlens, num_seqs, seqlen, reinterpret_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  mi355attn::FwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o_acc = o_acc;
  p.lse_acc = lse_acc;
  p.o_out = static_cast<__bf16*>(o_out);
  p.accumulate = accumulate;
  p.few_rows_apart = 1;
  p.cu_seqlens = cu_seqlens;
  p.num_seqs = num_seqs;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.seqlen = seqlen;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  p.key_split = 1;
  const int ks = mi355attn::fwd_key_split(batch, hq, seqlen);
  if (workspace != nullptr && ks > 1) {
    p.key_split = ks;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          mi355attn::fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks));
  }
  return mi355attn::launched(mi355attn::run_fwd_bf16(p, reinterpret_cast<hipStream_t>(stream)),
                               reinterpret_cast<hipStream_t>(stream));
}

attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* descale_q,
                         const float* descale_k, const float* descale_v, void* o, float* lse, void* workspace,
                         int batch, int hq, int hkv, int seqlen, int head_dim, int causal,
                         const int32_t* cu_seqlens, int num_seqs, float scale, attn_stream_t stream) {
  if (!q8 || !k8 || !v8 || !descale_q || !descale_k || !descale_v || !o || !lse) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace && !aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(descale_q) & 3u) || (reinterpret_cast<uintptr_t>(descale_k) & 3u) ||
      (reinterpret_cast<uintptr_t>(descale_v) & 3u))
    return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_common(batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  st = validate_cu(cu_seqlens, num_seqs, seqlen, reinterpret_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  mi355attn::Fp8FwdParams p{};
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.v = static_cast<const uint8_t*>(v8);
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.descale_v = descale_v;
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.num_seqs = num_seqs;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.seqlen = seqlen;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale = scale;
  p.key_split = 1;
  const int ks = mi355attn::fwd_key_split(batch, hq, seqlen);
  if (workspace != nullptr && ks > 1) {
    p.key_split = ks;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          mi355attn::fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks));
  }
  return mi355attn::launched(mi355attn::run_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream)),
                               reinterpret_cast<hipStream_t>(stream));
}

attn_status attn_fwd_fp8_merge(const void* q8, const void* k8, const void* v8, const float* descale_q,
                               const float* descale_k, const float* descale_v, float* o_acc, float* lse_acc,
                               void* o_out, int accumulate, void* workspace, int batch, int hq, int hkv, int seqlen,
                               int head_dim, int causal, const int32_t* cu_seqlens, int num_seqs, float scale,
                               attn_stream_t stream) {
  if (!q8 || !k8 || !v8 || !descale_q || !descale_k || !descale_v || !o_acc || !lse_acc)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o_acc) || (o_out && !aligned16(o_out)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(descale_q) & 3u) || (reinterpret_cast<uintptr_t>(descale_k) & 3u) ||
      (reinterpret_cast<uintptr_t>(descale_v) & 3u) || (reinterpret_cast<uintptr_t>(lse_acc) & 3u))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace && !aligned16(workspace)) return ATTN_ERR_INVALID_ARGUMENT;
  if (accumulate != 0 && accumulate != 1) return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = check_common(batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  st = validate_cu(cu_seqlens, num_seqs, seqlen, reinterpret_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  mi355attn::Fp8FwdParams p{};
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.v = static_cast<const uint8_t*>(v8);
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.descale_v = descale_v;
  p.o_acc = o_acc;
  p.lse_acc = lse_acc;
  p.o_out = static_cast<__bf16*>(o_out);
  p.accumulate = accumulate;
  p.cu_seqlens = cu_seqlens;
  p.num_seqs = num_seqs;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.seqlen = seqlen;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale = scale;
  p.key_split = 1;
  const int ks = mi355attn::fwd_key_split(batch, hq, seqlen);
  if (workspace != nullptr && ks > 1) {
    p.key_split = ks;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          mi355attn::fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks));
  }
  return mi355attn::launched(mi355attn::run_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream)),
                               reinterpret_cast<hipStream_t>(stream));
}

attn_status attn_bwd_phases(unsigned phases, const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                            int batch, int hq, int hkv, int seqlen, int head_dim, int causal,
                            const int32_t* cu_seqlens, int num_seqs, float scale, attn_stream_t stream) {
  const attn_status st = mi355attn::bwd_check(phases, q, k, v, o, lse, dout, dq, dk, dv, workspace, true, batch, hq,
                                              hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  return mi355attn::bwd_launch(phases, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                               mi355attn::bwd_head_split(batch, hq, hkv, seqlen),
                               mi355attn::bwd_key_split(batch, hq, seqlen), batch, hq, hkv, seqlen, head_dim, causal,
                               cu_seqlens, num_seqs, scale, reinterpret_cast<hipStream_t>(stream));
}

size_t attn_bwd_fp8_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim) {
  const size_t bf = attn_bwd_workspace_bytes(batch, hq, hkv, seqlen, head_dim);
  if (bf == 0 || head_dim != 128) return 0;
  return mi355attn::bwd_fp8_ws_offset(batch, hq, hkv, seqlen, head_dim) + bf;
}

attn_status attn_bwd_fp8(const void* q8, const void* k8, const void* v8, const float* descale_q,
                         const float* descale_k, const float* descale_v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, void* workspace, int batch, int hq, int hkv,
                         int seqlen, int head_dim, int causal, const int32_t* cu_seqlens, int num_seqs, float scale,
                         attn_stream_t stream) {
  if (!q8 || !k8 || !v8 || !descale_q || !descale_k || !descale_v) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8)) return ATTN_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(descale_q) & 3u) || (reinterpret_cast<uintptr_t>(descale_k) & 3u) ||
      (reinterpret_cast<uintptr_t>(descale_v) & 3u))
    return ATTN_ERR_INVALID_ARGUMENT;
  // q, k, v of the bf16 checks stand for the widened copies in the workspace
  attn_status st = mi355attn::bwd_check(ATTN_BWD_ALL, q8, k8, v8, o, lse, dout, dq, dk, dv, workspace, true, batch,
                                        hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = validate_cu(cu_seqlens, num_seqs, seqlen, s);  // before the first launch
  if (st != ATTN_OK) return st;
  char* ws = static_cast<char*>(workspace);
  __bf16* qw = reinterpret_cast<__bf16*>(ws);
  __bf16* kw = reinterpret_cast<__bf16*>(ws + mi355attn::bwd_fp8_k_offset(batch, hq, seqlen, head_dim));
  __bf16* vw = reinterpret_cast<__bf16*>(ws + mi355attn::bwd_fp8_v_offset(batch, hq, hkv, seqlen, head_dim));
  void* bws = ws + mi355attn::bwd_fp8_ws_offset(batch, hq, hkv, seqlen, head_dim);
  const size_t nq = (size_t)batch * seqlen * hq * head_dim, nkv = (size_t)batch * seqlen * hkv * head_dim;
  st = mi355attn::hip_result(mi355attn::run_widen_fp8(static_cast<const uint8_t*>(q8), qw, nq, s));
  if (st == ATTN_OK) st = mi355attn::hip_result(mi355attn::run_widen_fp8(static_cast<const uint8_t*>(k8), kw, nkv, s));
  if (st == ATTN_OK) st = mi355attn::hip_result(mi355attn::run_widen_fp8(static_cast<const uint8_t*>(v8), vw, nkv, s));
  if (st != ATTN_OK) return st;
  return mi355attn::bwd_launch(ATTN_BWD_ALL, qw, kw, vw, o, lse, dout, dq, dk, dv, bws,
                               mi355attn::bwd_head_split(batch, hq, hkv, seqlen),
                               mi355attn::bwd_key_split(batch, hq, seqlen), batch, hq, hkv, seqlen, head_dim, causal,
                               cu_seqlens, num_seqs, scale, s, descale_q, descale_k, descale_v);
}

attn_status attn_merge(float* o_acc, float* lse_acc, const void* o_part, const float* lse_part, void* o_out,
                       int batch, int seqlen, int heads, int head_dim, int accumulate, attn_stream_t stream) {
  if (!o_acc || !lse_acc || !o_part || !lse_part) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(o_acc) || !aligned16(o_part) || (o_out && !aligned16(o_out))) return ATTN_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(lse_acc) & 3u) || (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (batch < 1 || seqlen < 1 || heads < 1 || head_dim < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (accumulate != 0 && accumulate != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * seqlen * heads * (head_dim / 8) > (long long)UINT32_MAX * 256) return ATTN_ERR_UNSUPPORTED;
  mi355attn::MergeParams p{};
  p.o_acc = o_acc;
  p.lse_acc = lse_acc;
  p.o_part = static_cast<const __bf16*>(o_part);
  p.lse_part = lse_part;
  p.o_out = static_cast<__bf16*>(o_out);
  p.batch = batch;
  p.seqlen = seqlen;
  p.heads = heads;
  p.head_dim = head_dim;
  p.accumulate = accumulate;
  return mi355attn::launched(mi355attn::run_merge(p, reinterpret_cast<hipStream_t>(stream)),
                               reinterpret_cast<hipStream_t>(stream));
}

attn_status attn_bwd_accumulate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, float* dq_acc, float* dk_acc, float* dv_acc, int accumulate,
                                void* workspace, int batch, int hq, int hkv, int seqlen, int head_dim, int causal,
                                const int32_t* cu_seqlens, int num_seqs, float scale, attn_stream_t stream) {
  if (accumulate != 0 && accumulate != 1) return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status st = mi355attn::bwd_check(ATTN_BWD_ALL, q, k, v, o, lse, dout, dq_acc, dk_acc, dv_acc, workspace,
                                              true, batch, hq, hkv, seqlen, head_dim, causal, cu_seqlens, num_seqs,
                                              scale);
  if (st != ATTN_OK) return st;
  return mi355attn::bwd_launch(ATTN_BWD_ALL, q, k, v, o, lse, dout, dq_acc, dk_acc, dv_acc, workspace,
                               mi355attn::bwd_head_split(batch, hq, hkv, seqlen),
                               mi355attn::bwd_key_split(batch, hq, seqlen), batch, hq, hkv, seqlen, head_dim, causal,
                               cu_seqlens, num_seqs, scale, reinterpret_cast<hipStream_t>(stream), nullptr, nullptr,
                               nullptr, accumulate);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, void* workspace, int batch, int hq, int hkv, int seqlen,
                     int head_dim, int causal, const int32_t* cu_seqlens, int num_seqs, float scale,
                     attn_stream_t stream) {
  return attn_bwd_phases(ATTN_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, workspace, batch, hq, hkv, seqlen, head_dim,
                         causal, cu_seqlens, num_seqs, scale, stream);
}

}  // extern "C"
