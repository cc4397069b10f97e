// Internal interface between the C ABI layer (attn_api.hip) and the kernel
// files. Argument checking happens before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_index.h"

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
  int key_split;      // shares of each query block's key tiles (1: no split)
  float* part_o;      // key_split > 1: fp32 partial O [ks][B][S][Hq][D], each normalised by its share's sum
  float* part_lse;    // key_split > 1: fp32 m + log2 l [ks][B][Hq][S] (-inf for a share without visible keys)
  // Ring merge (attn_fwd_merge), when o_acc is not null: the call's result is
  // folded into a running one instead of being written to o and lse.
  float* o_acc;     // fp32 [B][S][Hq][D], read if accumulate, then overwritten
  float* lse_acc;   // fp32 [B][Hq][S], natural log, the same
  __bf16* o_out;    // bf16 copy of the merged O, or null
  int accumulate;   // 0: the running result starts empty
  int few_rows_apart;  // ring merge: rows with < 64 visible keys are merged by the few-key kernel (bf16 path)
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
  int key_split;    // as in FwdParams (1: no split)
  float* part_o;    // key_split > 1: fp32 partial O [ks][B][S][Hq][D]
  float* part_lse;  // key_split > 1: fp32 m + log2 l [ks][B][Hq][S], in log2 units of the scores
  // Ring merge (attn_fwd_fp8_merge), when o_acc is not null: as in FwdParams
  float* o_acc;
  float* lse_acc;
  __bf16* o_out;
  int accumulate;
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
  float* delta;  // workspace [B, Hq, stat_stride]: Delta_i = dO_i . O_i (sum_j P_ij dP_ij with < 64 keys)
  float* lse2;   // workspace [B, Hq, stat_stride]: LSE_i * log2(e)
  int stat_stride;  // seqlen rounded up to kStatAlign; the padding holds zeros
  int* order;       // workspace: dK/dV work order [num_blk * head_split], then dQ's [num_dq_blk * key_split]
  float* part;      // workspace [2][head_split][B][S][Hkv][D] fp32 partial dK, dV (head_split > 1 only)
  float* dq_part;   // workspace [key_split][B][S][Hq][D] fp32 partial dQ (key_split > 1 only)
  int head_split;   // query heads of a GQA group split over this many dK/dV workgroups
  int key_split;    // visible key tiles of a query block split over this many dQ workgroups
  const int32_t* cu_seqlens;
  int num_seqs;
  int batch, hq, hkv, seqlen, head_dim;
  int causal;
  float scale;
  float scale_log2e;
  int num_blk;     // 128-row blocks along the sequence (dK/dV key blocks); set by the launcher
  int dq_waves;    // dQ block geometry: 4 (128-query blocks) or 8 (256-query blocks)
  int num_dq_blk;  // dQ query blocks of 32 * dq_waves rows; set by the launcher
  // fp8 inputs (null for bf16): q, k, v then hold the E4M3 codes widened to
  // bf16 (exact), and the real inputs are code * descale. The kernels fold the
  // descales into their constants (scores, Delta and the dK, dQ outputs).
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  // attn_bwd_accumulate, when dq_acc is not null: fp32 dQ, dK, dV [shapes of
  // q, k, v] that the gradients are added to (accumulate = 1) or written to
  // (accumulate = 0) instead of the bf16 outputs
  float* dq_acc;
  float* dk_acc;
  float* dv_acc;
  int accumulate;
};

// Forward block geometry, picked from the sizes (the tiling matched to the
// sequence length of the FA-3 paragraph of the FlashAttention page): 4 waves
// of 32 queries (128-query blocks, two workgroups per CU) or 8 waves
// (256-query blocks, one per CU, each K/V tile copied into LDS once per CU
// instead of twice). Both give bitwise the same results. Taller blocks cost
// more masked work on the causal diagonal and at segment boundaries and fill
// the CUs less evenly; with D = 64 the 4-wave kernel also runs four waves per
// SIMD. Measured on MI355X (B * S = 32768 tokens, Hq = 28, Hkv = 4), time of
// 8 waves over 4:
//   D = 128 causal:     S = 2048 1.00, 4096 0.93, 8192 0.99, 16384 0.98, 32768 0.98
//   D = 128 non-causal: S = 2048 0.95, 4096 0.85, 8192 0.97, 16384 0.97, 32768 0.97
//   D = 64:             1.09 - 1.37 at every S, both masks
//   other shapes (D = 128): B=2 Hq=Hkv=32 S=8192 causal 1.00, non-causal 0.96;
//   B=4 Hq=Hkv=32 S=4096 causal 1.08; B=8 Hq=Hkv=32 S=2048 non-causal 0.94;
//   packed (Hq 14, Hkv 2, seed-4 lengths) causal 1.01, non-causal 1.00
// so 8 waves are taken for D = 128 without packing from S = 16384 (causal),
// where they win on every shape measured, or S = 2048 (non-causal). The
// environment variable ATTN_FWD_WAVES=4 or 8 overrides the choice (for tests
// and tuning).
int fwd_block_waves_env();  // 0 when unset
inline int fwd_block_waves(int seqlen, int head_dim, int causal, bool packed) {
  const int forced = fwd_block_waves_env();
  if (forced == 4 || forced == 8) return forced;
  if (packed || head_dim != 128) return 4;
  return seqlen >= (causal ? 16384 : 2048) ? 8 : 4;
}
// The dQ pass's block height, the same choice for the backward: 128 queries
// (4 waves, two workgroups per CU) or 256 (8 waves, one per CU, each K/V
// tile copied into LDS once per CU). Measured on MI355X (B * S = 32768
// tokens, Hq = 28, Hkv = 4), dQ time of 8 waves over 4:
//   D = 128 causal:     S = 2048 1.09, 4096 1.02, 8192 1.00, 16384 0.99, 32768 0.99
//   D = 128 non-causal: S = 2048 1.00, 4096 0.97, 8192 0.98, 16384 0.98, 32768 0.97
//   D = 64:             1.03 - 1.35 at every S, both masks
//   packed32k (Hq 14, Hkv 2, seed-4 lengths): causal 1.04, non-causal 1.02;
//   B=2 Hq=Hkv=32 S=8192 causal 1.02
// so 8 waves are taken for D = 128 without packing or key split from
// S = 16384 (causal) or S = 4096 (non-causal). ATTN_DQ_WAVES=4 or 8
// overrides it (for tests and tuning; a split dQ always runs 4 waves). The
// Delta phase, which writes the dQ work order, and the dQ phase must see the
// same choice.
int bwd_dq_waves_env();  // 0 when unset
inline int bwd_dq_block_waves(int seqlen, int head_dim, int causal, bool packed, int key_split) {
  if (key_split > 1) return 4;
  const int forced = bwd_dq_waves_env();
  if (forced == 4 || forced == 8) return forced;
  if (packed || head_dim != 128) return 4;
  return seqlen >= (causal ? 16384 : 4096) ? 8 : 4;
}
// The fp8 forward's block height: 128 queries (4 waves) or 256 (8 waves), same override.
inline int fwd_fp8_block_waves(int seqlen, int causal, bool packed) {
  const int forced = fwd_block_waves_env();
  if (forced == 4 || forced == 8) return forced;
  (void)seqlen;
  (void)causal;
  (void)packed;
  return 4;
}
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
// Combine the key-split partials of p.part_o / p.part_lse into p.o and p.lse
// (uses o, lse, part_o, part_lse, batch, seqlen, hq, head_dim, key_split).
hipError_t run_fwd_combine(const FwdParams& p, hipStream_t stream);
hipError_t run_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);
constexpr unsigned kBwdDelta = 1u, kBwdDkDv = 2u, kBwdDq = 4u;
hipError_t run_bwd(const BwdParams& p, unsigned phases, hipStream_t stream);
hipError_t run_merge(const MergeParams& p, hipStream_t stream);
// E4M3 codes -> bf16 (exact), n bytes from src to n bf16 values at dst.
hipError_t run_widen_fp8(const uint8_t* src, __bf16* dst, size_t n, hipStream_t stream);

// ATTN_OK for hipSuccess; otherwise records e for attn_last_hip_error() and
// returns ATTN_ERR_HIP.
attn_status hip_result(hipError_t e);
// hip_result of a call's last launch. Debug builds (ATTN_DEBUG) then
// synchronise `stream`, read and clear every kernel file's LDS fault word
// and return ATTN_ERR_DEBUG_CHECK if one was set.
attn_status launched(hipError_t e, hipStream_t stream);
#ifdef ATTN_DEBUG
// Each kernel file's LDS fault word, read and cleared (synchronous copies).
hipError_t lds_faults_fwd(unsigned int* out);
hipError_t lds_faults_fp8(unsigned int* out);
hipError_t lds_faults_bwd(unsigned int* out);
hipError_t lds_faults_merge(unsigned int* out);
#endif

// Argument checks shared by the backward entry points (no HIP call); a
// workspace pointer is required only when need_workspace is set.
attn_status bwd_check(unsigned phases, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, const void* workspace, bool need_workspace,
                      int batch, int hq, int hkv, int seqlen, int head_dim, int causal, const int32_t* cu_seqlens,
                      int num_seqs, float scale);
// Validation of cu_seqlens under ATTN_VALIDATE=1 (a copy and a sync), then
// the backward kernels with the given splits on a workspace laid out for
// them. Arguments must have passed bwd_check.
attn_status bwd_launch(unsigned phases, const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* workspace, int head_split, int key_split,
                       int batch, int hq, int hkv, int seqlen, int head_dim, int causal, const int32_t* cu_seqlens,
                       int num_seqs, float scale, hipStream_t stream, const float* descale_q = nullptr,
                       const float* descale_k = nullptr, const float* descale_v = nullptr, int accumulate = -1);
// accumulate >= 0: dq, dk, dv are fp32 arrays the gradients are added to (1)
// or written to (0) instead of bf16 outputs (attn_bwd_accumulate).

// fp8 backward workspace: the bf16 copies of the E4M3 codes of Q, K and V,
// each 256-byte aligned, then the bf16 backward's workspace.
inline size_t bwd_fp8_k_offset(int batch, int hq, int seqlen, int head_dim) {
  return align256((size_t)2 * batch * seqlen * hq * head_dim);
}
inline size_t bwd_fp8_v_offset(int batch, int hq, int hkv, int seqlen, int head_dim) {
  return bwd_fp8_k_offset(batch, hq, seqlen, head_dim) + align256((size_t)2 * batch * seqlen * hkv * head_dim);
}
inline size_t bwd_fp8_ws_offset(int batch, int hq, int hkv, int seqlen, int head_dim) {
  return bwd_fp8_v_offset(batch, hq, hkv, seqlen, head_dim) + align256((size_t)2 * batch * seqlen * hkv * head_dim);
}

}  // namespace mi355attn
