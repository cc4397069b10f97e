// Index arithmetic of the gfx950 attention kernels: LDS tile layouts and the
// per-lane addresses of every fragment read and tile copy, segment bounds,
// work shares. Plain integer functions, inlined into the kernels and also
// compiled for the host, where tests/index_check.cpp replays them over the
// kernels' whole index space (bounds, exact tile coverage, and the logical
// element every MFMA operand slot receives).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __HIP__
#define ATTN_HD __host__ __device__ inline
#else
#define ATTN_HD inline
#endif

namespace mi355attn {

ATTN_HD int imin(int a, int b) { return a < b ? a : b; }
ATTN_HD int imax(int a, int b) { return a > b ? a : b; }

// The LDS access rule of the debug build (-DATTN_DEBUG): an access of
// `bytes` bytes at LDS byte address `addr` must lie inside the workgroup's
// allocation of `size` bytes and be aligned to `align` (a power of two).
ATTN_HD bool lds_access_ok(uint32_t addr, uint32_t bytes, uint32_t align, uint32_t size) {
  return (addr & (align - 1u)) == 0u && addr <= size && bytes <= size - addr;
}

// Rows that see fewer than 64 keys: the first 63 rows of a causal segment of
// `len` rows, every row of a shorter non-causal segment. They are rows
// [0, n) of the segment, n = few_key_rows(len, causal), and see at most keys
// [0, n) of it; the tiled kernels leave them to the one-wave-per-row kernels.
constexpr int kFewKeyLimit = 64;
ATTN_HD int few_key_rows(int len, bool causal) {
  return causal ? imin(kFewKeyLimit - 1, len) : (len < kFewKeyLimit ? len : 0);
}

// Swap bits 2 and 3 of a row index in [0, 32): the K (or Q, dO) row a lane
// loads for the score product, so that C-layout register r of lane half h
// holds key 16 * (r / 8) + 8 * h + r % 8.
ATTN_HD int perm_rows(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Key offset (within a 32-key block) of C-layout register r of lane half h
// when the rows were loaded through perm_rows.
ATTN_HD int c_key(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

// ---------------------------------------------------------------------------
// LDS tile layouts: row-major [rows][D] bf16 with XOR swizzles of 16-byte
// chunks (each an involution, so the copy into LDS fetches, for physical
// chunk c of a row, the logical chunk swz(row, c)).
//
// "B128" tiles are read with 16-byte reads: lane l reads row perm_rows(l % 32)
// (+32 per block) at chunk 2t + l / 32. The swizzle permutes 16-byte chunks
// so that any 8 or 16 consecutive lanes hit distinct banks.
// "TR" tiles are read with transposing 8-byte reads (4 rows x 16 columns per
// 16 lanes). The swizzle permutes 8-byte units with a 4-row period.
// "Dual" tiles serve both kinds of read.
// ---------------------------------------------------------------------------

template <int D>
ATTN_HD int swz_b128(int row, int chunk) {
  if constexpr (D == 128) {
    const int f = (row & 3) | (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 3);
    return chunk ^ f;
  } else {
    const int f = ((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row ^ (row >> 2)) & 1) << 2);
    return chunk ^ f;
  }
}

// 8-byte unit XOR pattern for TR tiles, in units of 16-byte chunks (>> 1).
template <int D>
ATTN_HD int swz_tr_chunk(int row, int chunk) {
  // unit XOR table {0, 12, 24, 20} (8-byte units), halved to 16-byte chunks
  // {0, 6, 12, 10}, looked up by shifting a packed byte table (no branches)
  int x = (0x0A0C0600 >> (8 * (row & 3))) & 0xFF;
  if constexpr (D == 64) x &= 7;
  return chunk ^ x;
}

// One layout for tiles read both with 16-byte reads (rows through perm_rows)
// and with transposing reads (4 consecutive rows): the chunk XOR spreads 16
// consecutive rows over 16 chunks and 4 consecutive rows over 4 chunk groups.
template <int D>
ATTN_HD int swz_dual(int row, int chunk) {
  if constexpr (D == 128) {
    return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    // bits: row bit 1, row bit 2, row bit 1 ^ row bit 3
    return chunk ^ (((row >> 1) & 3) | ((((row >> 1) ^ (row >> 3)) & 1) << 2));
  }
}

// Element offset of (row, 16-byte chunk) or (row, 8-byte unit) in a tile.
template <int D>
ATTN_HD int off_b128(int row, int chunk) { return row * D + swz_b128<D>(row, chunk) * 8; }
template <int D>
ATTN_HD int off_tr_unit(int row, int unit) { return row * D + swz_tr_chunk<D>(row, unit >> 1) * 8 + (unit & 1) * 4; }
template <int D>
ATTN_HD int off_dual(int row, int chunk) { return row * D + swz_dual<D>(row, chunk) * 8; }
template <int D>
ATTN_HD int off_dual_unit(int row, int unit) { return row * D + swz_dual<D>(row, unit >> 1) * 8 + (unit & 1) * 4; }

// ---------------------------------------------------------------------------
// Tile copies (buffer_load ... lds): instruction i of wave w of a workgroup
// of W waves writes 16 bytes per lane at element (i W + w) 512 + 8 lane of
// the tile, which holds logical row e / D, logical chunk swz(row, physical
// chunk); the source is that chunk of that row in global memory, rows
// `stride` elements apart. Byte offsets within the tile's buffer range.
// ---------------------------------------------------------------------------
ATTN_HD int tile_dma_elem(int i, int waves, int wave, int lane) { return (i * waves + wave) * 512 + lane * 8; }
template <int D>
ATTN_HD uint32_t dma_src_b128(int e, int stride) {
  const int row = e / D;
  return (uint32_t)(row * stride + swz_b128<D>(row, (e % D) / 8) * 8) * 2u;
}
template <int D>
ATTN_HD uint32_t dma_src_tr(int e, int stride) {
  const int row = e / D;
  return (uint32_t)(row * stride + swz_tr_chunk<D>(row, (e % D) / 8) * 8) * 2u;
}
template <int D>
ATTN_HD uint32_t dma_src_dual(int e, int stride) {
  const int row = e / D;
  return (uint32_t)(row * stride + swz_dual<D>(row, (e % D) / 8) * 8) * 2u;
}

// ---------------------------------------------------------------------------
// Fragment reads of the 32x32x16 bf16 MFMA (lane l = (n, h), n = l % 32,
// h = l / 32).
// ---------------------------------------------------------------------------
// Row fragment of 32 rows x 16 columns (A operand, or B with rows as
// columns): lane reads row perm_rows(n), columns 16 t + 8 h .. + 7, of a B128
// tile (K in the forward, V in dQ) or a dual tile (Q, dO in dK/dV; K in dQ).
template <int D>
ATTN_HD int row_frag_b128(int lane, int t) { return off_b128<D>(perm_rows(lane & 31), 2 * t + (lane >> 5)); }
template <int D>
ATTN_HD int row_frag_dual(int lane, int t) { return off_dual<D>(perm_rows(lane & 31), 2 * t + (lane >> 5)); }
// Transposed fragment X^T (32 columns of X x 16 rows of X) from two
// transposing reads, rows 8 h + (l % 16) / 4 and + 4, 8-byte unit
// 8 c + 4 ((l / 16) % 2) + l % 4 for the 32-column block c; the reads of
// rows 16 u further add 16 u D.
template <int D>
ATTN_HD int tr_frag_tr(int lane, int c, int hi) {
  return off_tr_unit<D>(8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * hi, 8 * c + 4 * ((lane >> 4) & 1) + (lane & 3));
}
template <int D>
ATTN_HD int tr_frag_dual(int lane, int c, int hi) {
  return off_dual_unit<D>(8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * hi, 8 * c + 4 * ((lane >> 4) & 1) + (lane & 3));
}

// ---------------------------------------------------------------------------
// fp8 forward tiles: 64 rows x 128 bytes, XOR swizzles of 16-byte chunks.
// ---------------------------------------------------------------------------
// K tile: chunk c of row r at c ^ fk(r), where fk spreads the 8 even and the
// 8 odd rows of every 16 that one 16-lane group reads over 8 chunk positions.
ATTN_HD int fp8_fk_swz(int row) { return (row >> 1) & 7; }
// V tile: chunk c of row r at c ^ (r & 7): the 8 rows of one transposing read
// then cover all 32 banks.
ATTN_HD int fp8_fv_swz(int row) { return row & 7; }
// Tile copy: instruction i of wave w writes 16 bytes per lane at byte
// (i W + w) 1024 + 16 lane; source byte offsets within the buffer range.
ATTN_HD int fp8_dma_byte(int i, int waves, int wave, int lane) { return (i * waves + wave) * 1024 + lane * 16; }
ATTN_HD uint32_t fp8_dma_src_k(int off, int stride) {
  const int row = off / 128;
  return (uint32_t)(row * stride + (((off % 128) / 16) ^ fp8_fk_swz(row)) * 16);
}
ATTN_HD uint32_t fp8_dma_src_v(int off, int stride) {
  const int row = off / 128;
  return (uint32_t)(row * stride + (((off % 128) / 16) ^ fp8_fv_swz(row)) * 16);
}
// K row fragment of the 32x32x64 fp8 MFMA: lane reads bytes 64 t + 32 h + 16 i
// .. + 15 of row perm_rows(n) (i = 0, 1).
ATTN_HD int fp8_k_frag(int lane, int t, int i) {
  const int krow = perm_rows(lane & 31);
  return krow * 128 + ((4 * t + 2 * (lane >> 5) + i) ^ fp8_fk_swz(krow)) * 16;
}
// Source address of lane l for ds_read_b64_tr_b8 of the V^T fragment of the
// 32-column block db, key step 0: row 8 h + (l % 16) / 2, 8 bytes at
// 16 (2 db + (l / 16) % 2) + 8 (l % 2); key step q adds 16 q rows.
ATTN_HD int fp8_v_frag(int lane, int db) {
  const int g = (lane >> 4) & 1;
  const int s = lane & 15;
  const int row = 8 * (lane >> 5) + (s >> 1);
  return row * 128 + ((2 * db + g) ^ fp8_fv_swz(row)) * 16 + 8 * (s & 1);
}

// ---------------------------------------------------------------------------
// Segments and shares
// ---------------------------------------------------------------------------
// Segment [start, end) of token i for packed sequences (binary search over
// the prefix sums cu[0..n]); the whole sequence when cu is null.
ATTN_HD void segment_of(const int32_t* cu, int n, int seqlen, int i, int& start, int& end) {
  if (cu == nullptr) {
    start = 0;
    end = seqlen;
    return;
  }
  int lo = 0, hi = n;  // invariant: cu[lo] <= i < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid;
  }
  // Clamped so that 0 <= start <= i < end <= seqlen holds for any array:
  // a no-op for valid prefix sums, and a malformed one still keeps every
  // tile range inside the sequence.
  start = imax(0, imin(cu[lo], i));
  end = imin(seqlen, imax(cu[hi], i + 1));
}

// Items [lo, hi) of n handled by share `split` of `ns` (query heads of a
// group in the dK/dV pass, key tiles of a query block in the dQ pass and the
// forward key split).
ATTN_HD void share_range(int n, int ns, int split, int& lo, int& hi) {
  lo = split * n / ns;
  hi = (split + 1) * n / ns;
}

// ---------------------------------------------------------------------------
// Work splits and workspace layouts (host side)
// ---------------------------------------------------------------------------
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
// Workspace layout: partial O, then (256-byte aligned) the partial row statistics.
inline size_t fwd_part_lse_offset(int batch, int hq, int seqlen, int head_dim, int ks) {
  return align256((size_t)4 * ks * batch * seqlen * hq * head_dim);
}
inline size_t fwd_workspace_size(int batch, int hq, int seqlen, int head_dim) {
  const int ks = fwd_key_split(batch, hq, seqlen);
  if (ks == 1) return 0;
  return fwd_part_lse_offset(batch, hq, seqlen, head_dim, ks) + (size_t)4 * ks * batch * hq * seqlen;
}


}  // namespace mi355attn
