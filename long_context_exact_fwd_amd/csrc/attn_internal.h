// Internal interface between the C ABI layer (attn_api.hip) and the kernel
// files. Argument checking happens before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn.h"

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
  int* order;       // workspace: dK/dV work order [num_blk * head_split], then dQ's [num_blk * key_split]
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
  int num_blk;  // 128-row blocks along the sequence; set by the launcher
};

// Row length of the backward's per-row statistics in the workspace.
constexpr int kStatAlign = 64;
inline int stat_stride_for(int seqlen) { return (seqlen + kStatAlign - 1) / kStatAlign * kStatAlign; }

// dK/dV work split. The pass runs one workgroup of 8 waves per CU and per
// (b, kv head, 128-key block); with few kv heads and short sequences that is
// too few workgroups to fill the CUs and balance the causal costs. The G
// query heads of a group are then split over up to G workgroups, which write
// fp32 partial sums that a small kernel adds up.
constexpr long kDkdvTargetBlocks = 1024;  // about four workgroups per CU
inline int bwd_head_split(int batch, int hq, int hkv, int seqlen) {
  const long units = (long)batch * hkv * ((seqlen + 127) / 128);
  const int g = hq / hkv;
  if (units >= kDkdvTargetBlocks) return 1;
  const long want = (kDkdvTargetBlocks + units - 1) / units;
  return (int)(want < g ? want : g);
}
// dQ work split, for the same reason: the dQ pass runs two 4-wave
// workgroups per CU and per (b, query head, 128-query block); below about
// 1024 of them the visible key tiles of each block are split over up to 4
// workgroups, which write fp32 partial dQ.
inline int bwd_key_split(int batch, int hq, int seqlen) {
  const long units = (long)batch * hq * ((seqlen + 127) / 128);
  if (units >= kDkdvTargetBlocks) return 1;
  const long want = (kDkdvTargetBlocks + units - 1) / units;
  return (int)(want < 4 ? want : 4);
}
// Workspace layout, in bytes from its start: Delta and LSE*log2(e) (fp32
// [B, Hq, S64] each), the work order (int32, NB * (hs + ks) with
// NB = ceil(S / 128), hs and ks the head and key splits), then, each 256-byte
// aligned, the fp32 partial dK/dV and the fp32 partial dQ when their splits
// are above 1.
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline size_t bwd_order_offset(int batch, int hq, int seqlen) {
  return (size_t)8 * batch * hq * stat_stride_for(seqlen);
}
inline size_t bwd_part_offset(int batch, int hq, int seqlen, int hs, int ks) {
  const size_t nblk = ((size_t)seqlen + 127) / 128;
  return align256(bwd_order_offset(batch, hq, seqlen) + 4 * nblk * (size_t)(hs + ks));
}
inline size_t bwd_dq_part_offset(int batch, int hq, int hkv, int seqlen, int head_dim, int hs, int ks) {
  const size_t part = hs > 1 ? (size_t)8 * hs * batch * seqlen * hkv * head_dim : 0;
  return align256(bwd_part_offset(batch, hq, seqlen, hs, ks) + part);
}
inline size_t bwd_workspace_size(int batch, int hq, int hkv, int seqlen, int head_dim, int hs, int ks) {
  const size_t part = ks > 1 ? (size_t)4 * ks * batch * seqlen * hq * head_dim : 0;
  return bwd_dq_part_offset(batch, hq, hkv, seqlen, head_dim, hs, ks) + part;
}
// ... with the splits chosen from the sizes
inline size_t bwd_workspace_size(int batch, int hq, int hkv, int seqlen, int head_dim) {
  return bwd_workspace_size(batch, hq, hkv, seqlen, head_dim, bwd_head_split(batch, hq, hkv, seqlen),
                            bwd_key_split(batch, hq, seqlen));
}

// Forward key split. The forward runs one workgroup per (b, query head,
// 128-query block), two per CU, and a block's time grows with the keys it
// visits. One workgroup alone on a CU still reaches about 94 % of the
// throughput of two, so what a small grid loses is the slowest block (the last
// one under a causal mask, twice the average) running on while CUs idle: with
// fewer than about 512 blocks it outlasts the per-CU share of the work. The
// key tiles of each block are then split over up to 8 workgroups; each writes
// an fp32 partial (O normalised by its own sum, and m + log2 l), and a second
// kernel combines the shares. Every share keeps at least 32 key tiles (2048
// keys): the combine moves 8 bytes per share and output element, which
// shorter rows do not earn back. The split needs the caller's workspace;
// without one the forward runs unsplit.
constexpr long kFwdTargetBlocks = 512;
constexpr int kFwdMaxKeySplit = 8;
constexpr int kFwdMinTilesPerShare = 32;
inline int fwd_key_split(int batch, int hq, int seqlen) {
  const long units = (long)batch * hq * ((seqlen + 127) / 128);
  if (units >= kFwdTargetBlocks) return 1;
  long ks = (kFwdTargetBlocks + units - 1) / units;
  if (ks > kFwdMaxKeySplit) ks = kFwdMaxKeySplit;
  const long by_len = ((long)seqlen + 63) / 64 / kFwdMinTilesPerShare;
  if (ks > by_len) ks = by_len;
  return ks < 1 ? 1 : (int)ks;
}
// Forward block geometry, picked from the sizes (the tiling matched to the
// sequence length of the FA-3 paragraph of the FlashAttention page): 4 waves
// of 32 queries (128-query blocks, two workgroups per CU) or 8 waves
// (256-query blocks, one per CU, each K/V tile copied into LDS once per CU
// instead of twice). Both give bitwise the same results. Taller blocks cost
// more masked work on the causal diagonal and at segment boundaries and fill
// the CUs less evenly; with D = 64 the 4-wave kernel (161 VGPRs) also runs
// three waves per SIMD against two. Measured on MI355X (B * S = 32768 tokens,
// Hq = 28, Hkv = 4), time of 8 waves over 4:
//   D = 128 causal:     S = 2048 1.11, 4096 0.98, 8192 1.01, 16384 1.00, 32768 0.99
//   D = 128 non-causal: S = 2048 0.99, 4096 0.92, 8192 0.97, 16384 0.98, 32768 0.97
//   D = 64:             1.10 - 1.35 at every S, both masks
//   packed (Hq 14, Hkv 2, seed-4 lengths): D = 128 1.07, D = 64 1.20
// so 8 waves are taken for D = 128 without packing from S = 16384 (causal) or
// S = 4096 (non-causal). The environment variable ATTN_FWD_WAVES=4 or 8
// overrides the choice (for tests and tuning).
int fwd_block_waves_env();  // 0 when unset
inline int fwd_block_waves(int seqlen, int head_dim, int causal, bool packed) {
  const int forced = fwd_block_waves_env();
  if (forced == 4 || forced == 8) return forced;
  if (packed || head_dim != 128) return 4;
  return seqlen >= (causal ? 16384 : 4096) ? 8 : 4;
}
// Workspace layout: partial O, then (256-byte aligned) the partial row statistics.
inline size_t fwd_part_lse_offset(int batch, int hq, int seqlen, int head_dim, int ks) {
  return align256((size_t)4 * ks * batch * seqlen * hq * head_dim);
}
inline size_t fwd_workspace_size(int batch, int hq, int seqlen, int head_dim) {
  const int ks = fwd_key_split(batch, hq, seqlen);
  if (ks == 1) return 0;
  return fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks) + (size_t)4 * ks * batch * hq * seqlen;
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

// ATTN_OK for hipSuccess; otherwise records e for attn_last_hip_error() and
// returns ATTN_ERR_HIP.
attn_status hip_result(hipError_t e);

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
                       int num_seqs, float scale, hipStream_t stream);

}  // namespace mi355attn
