/*
 * attn.h: C ABI of the MI355X (gfx950) exact-attention library libmi355attn.so.
 *
 * What it computes. Exact scaled-dot-product attention
 *     O = softmax(Q K^T * scale + mask) V
 * computed tile by tile with an online softmax, so the S x S score matrix is
 * never written to device memory. Sources:
 *   - "ms-swift集成FlashAttention 2/3，长文本训练更高效", section
 *     "FlashAttention 如何破局": Q, K and V are split along the sequence; each
 *     workgroup holds a Q block on chip and streams the matching K/V blocks;
 *     QK^T, softmax and PV stay on chip, a running maximum and normaliser are
 *     kept per row, and only the output goes back to global memory.
 *   - The same page's section on why standard attention is memory-hungry
 *     defines the unfused computation this must equal (QK^T, softmax, PV over
 *     a [B, H, S, S] tensor).
 *   - The backward recomputes the probabilities from the saved log-sum-exp;
 *     the same memory section notes that the backward needs the intermediates
 *     again.
 * The shapes are one GPU's share of Ulysses sequence parallelism
 * ("ms-swift长文本训练秘诀：Ulysses并行技术解析" §1; FlashAttention page, the
 * Ulysses part of the sequence-parallel section): after the all-to-all a GPU
 * holds the full sequence for a subset of heads. Nothing here communicates.
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers unless stated. Tensors are contiguous and
 *     16-byte aligned. Q, O, dO, dQ are [B, S, Hq, D]; K, V, dK, dV are
 *     [B, S, Hkv, D]; LSE is float32 [B, Hq, S]: the natural-log
 *     log-sum-exp of each row's scaled, masked scores.
 *   - GQA: query head h reads key/value head h / (Hq / Hkv); Hq must be a
 *     multiple of Hkv.
 *   - Masks: causal means key j is visible to query i iff j <= i. With
 *     cu_seqlens (int32 device array of num_seqs + 1 prefix sums, first 0,
 *     strictly increasing, last == seqlen) the batch must be 1 and seqlen is
 *     the total packed length. Key j is then visible to query i only when
 *     both lie in the same segment (block-diagonal), and causal applies
 *     within the segment. Packing several samples into one long sequence is
 *     the packing of the Ulysses page §5 and of the FlashAttention page's
 *     section on engineering results. cu_seqlens contents are not checked
 *     by default (that needs a copy to the host and a sync): a malformed
 *     array gives meaningless results, but the kernels clamp every segment to
 *     [0, seqlen) around its own row, so they never access memory outside the
 *     tensors. With the environment variable ATTN_VALIDATE=1 each call copies
 *     cu_seqlens to the host first (synchronising `stream`) and returns
 *     ATTN_ERR_INVALID_ARGUMENT, with nothing launched, unless cu_seqlens[0]
 *     = 0, the entries strictly increase and cu_seqlens[num_seqs] = seqlen.
 *   - scale must be finite and > 0 (the configurations use 1/sqrt(D)).
 *   - head_dim must be 64 or 128 (bf16 paths) or 128 (fp8 path); other values
 *     return ATTN_ERR_UNSUPPORTED so the caller can fall back to a standard
 *     implementation. Automatic fallback when the fused kernel is unusable
 *     is described in the FlashAttention page's "实际怎么用" section.
 *   - Size: seqlen * Hq * D must not exceed 2^31 - 1 (the kernels address one
 *     batch slice with 32-bit row offsets and their tile copies with 32-bit
 *     byte ranges); larger requests return ATTN_ERR_UNSUPPORTED. attn_merge
 *     accepts up to 2^40 elements in total.
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     forward and backward workspaces. The library allocates nothing and keeps no state
 *     besides its loaded code. It is safe to call from several host threads.
 *   - Asynchrony: each call only enqueues kernels on `stream` (0 = the null
 *     stream). Results are valid once the stream reaches that point.
 *   - Errors: every argument check runs before any HIP call (ATTN_VALIDATE's
 *     copy comes after them). A non-OK status means nothing was enqueued,
 *     except ATTN_ERR_HIP, which reports a failed copy or launch
 *     (attn_last_hip_error() then gives the hipError_t value).
 *   - Determinism: no atomics; identical inputs give bitwise identical outputs.
 *   - Tiling: the kernels pick their block heights from the sizes (128- or
 *     256-query blocks for the forward and for the backward's dQ pass) and
 *     split small grids; every choice gives results within the stated
 *     tolerances, and the two block heights give bitwise the same results.
 *     The environment variables ATTN_FWD_WAVES=4|8 and ATTN_DQ_WAVES=4|8
 *     force the forward's and the dQ pass's block height (4 waves: 128
 *     queries; 8 waves: 256), for tests and tuning.
 *   - Debug build: libmi355attn_debug.so exports this same interface, built
 *     with -DATTN_DEBUG. Its kernels check each LDS access made through the
 *     library's access helpers (tile copies, fragment and statistics reads,
 *     the few-key kernel's rows) against the workgroup's LDS allocation and
 *     the access's alignment before issuing it, skip a failing access, and
 *     record it; each entry point then synchronises `stream` and returns
 *     ATTN_ERR_DEBUG_CHECK if any access failed. It gives bitwise the same
 *     outputs as this library and is much slower; it is meant for tests.
 */
#ifndef MI355ATTN_ATTN_H_
#define MI355ATTN_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* attn_stream_t; /* same object as hipStream_t */

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* inconsistent shape, flag or pointer; nothing enqueued */
  ATTN_ERR_UNSUPPORTED = 2,      /* valid request the library has no kernel for; caller may fall back */
  ATTN_ERR_HIP = 3,              /* a kernel launch failed; see attn_last_hip_error() */
  ATTN_ERR_SCRATCH_TOO_SMALL = 4, /* attn_bwd_noalloc: the request needs more than its fixed scratch; nothing enqueued */
  ATTN_ERR_DEBUG_CHECK = 5        /* debug build only: a kernel's LDS access check failed; outputs are invalid */
} attn_status;

/* Bytes of device workspace attn_fwd (and attn_fwd_fp8) can use for these sizes: 0 when the
 * forward runs unsplit. The FA-3 paragraph of the FlashAttention page (section
 * "那么FlashAttention-2 和 -3 又改进了什么") has the kernel pick its tiling from
 * the sequence length; here the work split is picked from the sizes. With
 * fewer than 512 (batch, query head, 128-query block) units the key tiles of
 * each block are split over ks = min(8, ceil(512 / units), ceil(seqlen/64)/32)
 * workgroups (ks > 1 needs 64 key tiles, seqlen > 4032). The workspace then holds fp32
 * partial O [ks, B, S, Hq, D] and, 256-byte aligned after it, fp32 partial row
 * statistics [ks, B, Hq, S]. Returns 0 for invalid sizes as well. */
size_t attn_fwd_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim);

/* Forward, bf16 in and out.
 * q [B,S,Hq,D], k and v [B,S,Hkv,D] bfloat16 (read only).
 * o [B,S,Hq,D] bfloat16 (written). lse [B,Hq,S] float32 (written).
 * workspace: NULL, or 16-byte aligned device memory of at least
 * attn_fwd_workspace_bytes() bytes, owned by the caller, contents on entry
 * ignored; calls that may run at the same time need separate workspaces. With
 * NULL the forward always runs one
 * workgroup per query block. With a workspace, sizes that
 * attn_fwd_workspace_bytes() sizes above 0 run the key split: each share
 * writes its partial output, and a second kernel combines the shares
 * (O = sum of the shares' O weighted by 2^(their m + log2 l) over the total).
 * Rounding: O is accumulated in fp32 and rounded to bf16 (nearest-even). The
 * probabilities enter the PV product rounded to bf16 (the row sum uses them
 * unrounded), except in rows that see fewer than 64 keys: a last small kernel
 * recomputes those rows in fp32 with unrounded probabilities.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                     int batch, int hq, int hkv, int seqlen, int head_dim,
                     int causal, const int32_t* cu_seqlens, int num_seqs,
                     float scale, attn_stream_t stream);

/* Forward with OCP FP8 E4M3FN inputs and per-tensor scales.
 * FP8 appears in the FA-3 paragraph of the FlashAttention page; per-tensor
 * scaling of E4M3 data appears in the Q-Galore section of
 * "ms-swift支持GPU显存碎片整理提升利用率".
 * q8, k8, v8: uint8 E4M3FN codes, shapes as q, k, v. The real inputs are
 * code * descale. descale_q/k/v: device pointers to one float each.
 * o: bfloat16 [B,S,Hq,D]; lse: float32 [B,Hq,S] of the dequantised scores.
 * The probabilities fed to the PV product are rounded to E4M3. The row sum is
 * taken from the fp32 probabilities. head_dim must be 128. workspace: as for
 * attn_fwd (NULL, or attn_fwd_workspace_bytes() bytes for the same sizes);
 * the key split and the combine work the same way.
 */
attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         void* o, float* lse, void* workspace,
                         int batch, int hq, int hkv, int seqlen, int head_dim,
                         int causal, const int32_t* cu_seqlens, int num_seqs,
                         float scale, attn_stream_t stream);

/* Bytes of device workspace attn_bwd needs for these sizes. It holds, in
 * order: two fp32 per-row arrays [batch, hq, S64] (S64 = seqlen rounded up to
 * a multiple of 64): Delta_i = dO_i . O_i (sum_j P_ij dP_ij in rows that see
 * fewer than 64 keys, all of them in this call) and LSE_i * log2(e), the
 * padding rows written as zeros; the int32 work order of the dK/dV and dQ
 * kernels (NB * (hsplit + ksplit) entries, NB = ceil(seqlen / 128)); then, each
 * 256-byte aligned, fp32 partial dK and dV (8 * hsplit * batch * seqlen * hkv
 * * head_dim bytes) when the dK/dV pass splits a GQA group's query heads over
 * hsplit > 1 workgroups, and fp32 partial dQ (4 * ksplit * batch * seqlen *
 * hq * head_dim bytes) when the dQ pass splits a query block's key tiles over
 * ksplit > 1 workgroups. Both splits are chosen from the sizes, for grids too
 * small to fill the GPU. Returns 0 for non-positive sizes, hq % hkv != 0 or
 * a request over the size limit above. */
size_t attn_bwd_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim);

/* Backward: dq, dk, dv from q, k, v, the forward's o and lse, and dout.
 * The probabilities are recomputed from lse. No S x S buffer is used.
 * Inputs are bf16 (lse float32); dq [B,S,Hq,D], dk and dv [B,S,Hkv,D] are
 * bf16 and fully overwritten. For GQA, dk and dv sum over the query heads of
 * each group. workspace: at least attn_bwd_workspace_bytes() bytes, 16-byte
 * aligned, owned by the caller, contents on entry ignored.
 * Three phases run on `stream` in order: Delta (one kernel for dO . O and
 * the work order, a second for the rows with fewer than 64 keys), dK/dV, dQ.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     int batch, int hq, int hkv, int seqlen, int head_dim,
                     int causal, const int32_t* cu_seqlens, int num_seqs,
                     float scale, attn_stream_t stream);

/* attn_bwd with fp32 gradient accumulators, for the backward of a
 * Ring-Attention forward: the gradients of one (query chunk, key chunk) pair,
 * computed as attn_bwd does from the final o and lse of the query chunk
 * (Ring-Attention paragraph of the FlashAttention page's sequence-parallel
 * section: the backward of a ring step is the same recomputation with the
 * given LSE), are added to running sums instead of being rounded to bf16.
 * dq_acc float32 [B,S,Hq,D], dk_acc and dv_acc float32 [B,S,Hkv,D], 16-byte
 * aligned: accumulate = 1 adds the pair's gradients to them, 0 overwrites
 * them (the first pair). Other arguments and the workspace as attn_bwd.
 * Every element of the three arrays is read and written by one thread, and
 * calls on the same arrays must be ordered (one stream). Rounded to bf16, the
 * result of accumulate = 0 equals attn_bwd's output bit for bit. */
attn_status attn_bwd_accumulate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, float* dq_acc, float* dk_acc, float* dv_acc, int accumulate,
                                void* workspace, int batch, int hq, int hkv, int seqlen, int head_dim,
                                int causal, const int32_t* cu_seqlens, int num_seqs,
                                float scale, attn_stream_t stream);

/* One or more of the three backward phases, in the fixed order Delta, dK/dV,
 * dQ: attn_bwd(...) is attn_bwd_phases(ATTN_BWD_ALL, ...). Running the
 * phases as separate calls on one stream (Delta first) gives bitwise the
 * same result. It exists so that callers and profilers can time or schedule
 * each phase on its own. Arguments as attn_bwd. dK/dV and dQ read the Delta
 * and the block order that an earlier ATTN_BWD_DELTA call left in `workspace`.
 * phases: nonzero bitmask of the values below; other bits are invalid. */
#define ATTN_BWD_DELTA 1u
#define ATTN_BWD_DKDV 2u
#define ATTN_BWD_DQ 4u
#define ATTN_BWD_ALL 7u
attn_status attn_bwd_phases(unsigned phases, const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                            int batch, int hq, int hkv, int seqlen, int head_dim,
                            int causal, const int32_t* cu_seqlens, int num_seqs,
                            float scale, attn_stream_t stream);

/* Backward of attn_fwd_fp8: dq, dk, dv (bf16) of attention over the
 * dequantised inputs Q = q8 * descale_q, K = k8 * descale_k,
 * V = v8 * descale_v, from the forward's o (bf16) and lse and the upstream
 * gradient dout (bf16). FP8 is named in the FA-3 paragraph of the
 * FlashAttention page ("那么FlashAttention-2 和 -3 又改进了什么"), per-tensor
 * scaling of E4M3 data in the Q-Galore section of
 * "ms-swift支持GPU显存碎片整理提升利用率"; the pages give no FP8 backward,
 * so this one is the exact gradient of the forward's definition.
 * An E4M3 code is exact in bf16, so a first kernel widens q8, k8, v8 to bf16
 * copies in the workspace and the bf16 backward kernels run on them with the
 * descales folded into their constants (scores: scale * d_q * d_k; Delta
 * divided by d_v; dK times scale * d_q * d_v; dQ times scale * d_k * d_v).
 * Arguments as attn_fwd_fp8 and attn_bwd; head_dim must be 128. workspace: at
 * least attn_bwd_fp8_workspace_bytes() bytes, 16-byte aligned, owned by the
 * caller: the bf16 copies of q, k, v (each 256-byte aligned) and then the
 * workspace attn_bwd uses. Returns 0 for unsupported sizes. */
size_t attn_bwd_fp8_workspace_bytes(int batch, int hq, int hkv, int seqlen, int head_dim);
attn_status attn_bwd_fp8(const void* q8, const void* k8, const void* v8,
                         const float* descale_q, const float* descale_k, const float* descale_v,
                         const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* workspace,
                         int batch, int hq, int hkv, int seqlen, int head_dim,
                         int causal, const int32_t* cu_seqlens, int num_seqs,
                         float scale, attn_stream_t stream);

/* Backward without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, allocation-free serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and results as
 * attn_bwd, minus the workspace: the workspace is a fixed array of
 * ATTN_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from
 * the first call on a device until the process ends. The call makes no
 * allocation of its own (its first call on a device looks up that device's
 * copy of the array).
 *   - The calling thread's current device must be the one `stream` runs on.
 *   - When attn_bwd_workspace_bytes() for these sizes exceeds the scratch,
 *     the backward runs without its head and key splits (the same kernels,
 *     one workgroup per GQA group and per query block; results then differ
 *     from attn_bwd's in rounding only). If even that needs more than the
 *     scratch (8 * batch * hq * S64 bytes plus the work order), it returns
 *     ATTN_ERR_SCRATCH_TOO_SMALL and enqueues nothing.
 *   - Every call on a device shares that device's scratch and leaves its
 *     contents behind (no call needs it cleared): calls that may run at the
 *     same time on one device (other streams, other threads) race and must be
 *     serialised by the caller. */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv,
                             int batch, int hq, int hkv, int seqlen, int head_dim,
                             int causal, const int32_t* cu_seqlens, int num_seqs,
                             float scale, attn_stream_t stream);

/* Ring-Attention step: merge one partial attention result into a running one.
 * Ring-Attention passes K/V blocks around a ring and accumulates partial
 * attention results locally (FlashAttention page, sequence-parallel section,
 * Ring-Attention paragraph; Ring-Attention section of
 * "ms-swift支持GPU显存碎片整理提升利用率"). Attention over two disjoint key
 * sets combines exactly into attention over their union:
 *   M = max(LSE_acc, LSE_part), w = e^(LSE - M) for each,
 *   O = (w_acc O_acc + w_part O_part) / (w_acc + w_part),
 *   LSE = M + ln(w_acc + w_part);
 * a part with LSE = -inf has weight 0; if both do, O = 0 and LSE = -inf.
 * o_acc: float32 [B,S,H,D] (read if accumulate, then overwritten with the
 * merged O). lse_acc: float32 [B,H,S] (same). accumulate = 0 treats the
 * running result as empty (first ring step: the merge copies the part).
 * o_part: bfloat16 [B,S,H,D] and lse_part float32 [B,H,S], e.g. attn_fwd's
 * outputs for one K/V block. o_out: bfloat16 [B,S,H,D] copy of the merged O
 * (nearest-even), or NULL. The four arrays must not overlap. Each element is
 * read and written by one thread, so o_acc/lse_acc are updated in place.
 * head_dim 64 or 128; o_acc, o_part, o_out 16-byte aligned. */
attn_status attn_merge(float* o_acc, float* lse_acc, const void* o_part, const float* lse_part, void* o_out,
                       int batch, int seqlen, int heads, int head_dim, int accumulate, attn_stream_t stream);

/* Ring-Attention step fused into the forward: the attention of q over this
 * call's k and v (the same function attn_fwd computes, with the same causal,
 * GQA and packing rules) is merged straight into a running result with the
 * attn_merge formula, so the partial never leaves the chip in bf16 and no
 * separate merge kernel runs. The ring itself (FlashAttention page,
 * sequence-parallel section, Ring-Attention paragraph) is the caller's: per
 * arriving K/V block, one call with accumulate = 1 (0 for the first block).
 * q, k, v: bfloat16, as for attn_fwd (read only).
 * o_acc: float32 [B,S,Hq,D], lse_acc: float32 [B,Hq,S] (natural log): read
 * if accumulate, then overwritten with the merged result. accumulate = 0
 * treats the running result as empty (its contents are not read).
 * o_out: bfloat16 [B,S,Hq,D] copy of the merged O (nearest-even), or NULL.
 * workspace: as for attn_fwd (NULL, or attn_fwd_workspace_bytes() bytes);
 * with a key split the combine kernel does the merge.
 * No array may overlap another. Rounding: the partial result stays fp32 up
 * to the merge; the bf16 probabilities in the PV product and the fp32
 * recomputation of rows that see fewer than 64 keys are as in attn_fwd.
 * Every element of o_acc and lse_acc is read and written by one wave, so the
 * update is in place; calls on one running result must be ordered (one
 * stream).
 */
attn_status attn_fwd_merge(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc, void* o_out,
                           int accumulate, void* workspace, int batch, int hq, int hkv, int seqlen, int head_dim,
                           int causal, const int32_t* cu_seqlens, int num_seqs, float scale, attn_stream_t stream);

/* attn_fwd_merge for the fp8 forward: the attention attn_fwd_fp8 computes
 * (E4M3 q8, k8, v8 with per-tensor descales, head_dim 128) merged into the
 * running fp32 (o_acc, lse_acc) in the forward's epilogue, with the formula,
 * arguments and workspace of attn_fwd_merge. The fp8 path has no fp32
 * recomputation of rows that see few keys: every row's probabilities enter
 * the PV product rounded to E4M3, as in attn_fwd_fp8.
 */
attn_status attn_fwd_fp8_merge(const void* q8, const void* k8, const void* v8,
                               const float* descale_q, const float* descale_k, const float* descale_v,
                               float* o_acc, float* lse_acc, void* o_out, int accumulate, void* workspace,
                               int batch, int hq, int hkv, int seqlen, int head_dim,
                               int causal, const int32_t* cu_seqlens, int num_seqs,
                               float scale, attn_stream_t stream);

/* Static string naming a status code ("ATTN_OK", ...). Never NULL. */
const char* attn_status_str(attn_status s);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355ATTN_ATTN_H_ */
