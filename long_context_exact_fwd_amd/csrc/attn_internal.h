// Internal interface between the C ABI layer (attn_api.hip) and the kernel
// files. Argument checking happens before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355attn {

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const int32_t* cu_seqlens;  // null when not packed
  int num_seqs;
  int batch, hq, hkv, seqlen, head_dim;
  int causal;
  float scale;
  float scale_log2e;  // scale * log2(e)
  int num_qblk;       // set by the launcher
};

struct Fp8FwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  __bf16* o;
  float* lse;
  const int32_t* cu_seqlens;
  int num_seqs;
  int batch, hq, hkv, seqlen, head_dim;
  int causal;
  float scale;
  int num_qblk;
};

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const float* lse;
  const __bf16* dout;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* delta;  // workspace [B, Hq, stat_stride]: Delta_i = dO_i . O_i
  float* lse2;   // workspace [B, Hq, stat_stride]: LSE_i * log2(e)
  int stat_stride;  // seqlen rounded up to kStatAlign; the padding holds zeros
  int* order;       // workspace [2, num_blk]: block order of the dK/dV pass, then of the dQ pass
  const int32_t* cu_seqlens;
  int num_seqs;
  int batch, hq, hkv, seqlen, head_dim;
  int causal;
  float scale;
  float scale_log2e;
  int num_blk;  // 128-row blocks along the sequence; set by the launcher
};

// Row length of the backward's per-row statistics in the workspace.
constexpr int kStatAlign = 64;
inline int stat_stride_for(int seqlen) { return (seqlen + kStatAlign - 1) / kStatAlign * kStatAlign; }

struct MergeParams {
  float* o_acc;            // [B, S, H, D] fp32, read if accumulate, written
  float* lse_acc;          // [B, H, S] fp32, read if accumulate, written
  const __bf16* o_part;    // [B, S, H, D] bf16
  const float* lse_part;   // [B, H, S] fp32
  __bf16* o_out;           // [B, S, H, D] bf16 or null
  int batch, seqlen, heads, head_dim;
  int accumulate;
};

hipError_t run_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t run_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);
constexpr unsigned kBwdDelta = 1u, kBwdDkDv = 2u, kBwdDq = 4u;
hipError_t run_bwd(const BwdParams& p, unsigned phases, hipStream_t stream);
hipError_t run_merge(const MergeParams& p, hipStream_t stream);

}  // namespace mi355attn
