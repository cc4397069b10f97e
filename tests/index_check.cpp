// Host replay of the attention kernels' index arithmetic (attn_index.h), built
// with g++ and run by tests/test_index_bounds.py.
//
// For every LDS tile the kernels use it simulates the tile copy (each lane's
// 16-byte DMA write and the global chunk it fetches) and every fragment read
// of every lane: each access must stay inside the tile, the copy must fill the
// tile exactly once with every logical element of the tile, and each MFMA
// operand slot must receive the logical element the product needs (rows
// through perm_rows for row fragments; the transposing reads' lane exchange
// for transposed fragments). It then sweeps sequence shapes for the tile
// ranges of the query and key blocks (every visible key of a row inside its
// block's range, the range inside the sequence, key-split shares disjoint and
// covering), the workspace layouts (aligned, ordered, disjoint, within the
// reported size) and the 32-bit byte ranges of the tile copies at the largest
// sequence the library accepts (seqlen * Hq * D = 2^31 - 1).
//
// LDS banks: every read must also be free of bank conflicts under this model
// of the gfx950 LDS: 64 banks of 4 bytes; a 16-byte read is served 16 lanes
// at a time and an 8-byte read (plain or transposing) 32 lanes at a time, and
// the lanes served together must touch distinct banks. Under the model the
// bf16 kernels' reads are conflict-free, which SQ_LDS_BANK_CONFLICT = 0 on
// MI355X confirms, and it flagged the 2-way conflicts of an earlier fp8 K tile
// layout, which that counter had shown.
//
// Exit status 0 and a last line "index_check: OK" when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <set>
#include <utility>
#include <vector>

#ifndef ATTN_INDEX_HEADER
#define ATTN_INDEX_HEADER "../long_context_exact_fwd_amd/csrc/attn_index.h"
#endif
#include ATTN_INDEX_HEADER

using namespace mi355attn;

static long g_checks = 0;
static int g_fail = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    ++g_checks;                                            \
    if (!(cond)) {                                         \
      if (g_fail < 20) {                                   \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        fprintf(stderr, __VA_ARGS__);                      \
        fprintf(stderr, "\n");                             \
      }                                                    \
      ++g_fail;                                            \
    }                                                      \
  } while (0)

// Logical (row, column) held by each element of a simulated LDS tile.
struct Tag {
  int row = -1, col = -1;
  bool operator==(const Tag& o) const { return row == o.row && col == o.col; }
};

enum Swz { kB128, kTR, kDual };

template <int D>
uint32_t dma_src(Swz swz, int e, int stride) {
  return swz == kB128 ? dma_src_b128<D>(e, stride) : swz == kTR ? dma_src_tr<D>(e, stride) : dma_src_dual<D>(e, stride);
}

// Fill a 64-row bf16 tile the way a workgroup of `waves` waves copies it.
template <int D>
std::vector<Tag> fill_tile(Swz swz, int waves, const char* what) {
  constexpr int TILE = 64 * D;
  const int ni = TILE * 2 / (waves * 1024);
  CHECK(ni * waves * 512 == TILE, "%s: copy instructions do not cover the tile", what);
  const int stride = 3 * D + 8;  // a row pitch unlike D, so a row/column mix-up shows
  std::vector<Tag> tile(TILE);
  for (int w = 0; w < waves; ++w)
    for (int i = 0; i < ni; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int e = tile_dma_elem(i, waves, w, lane);
        CHECK(e >= 0 && e + 8 <= TILE && e % 8 == 0, "%s: copy destination %d outside the tile", what, e);
        if (e < 0 || e + 8 > TILE) continue;
        // the wave's M0 base is the lane-0 destination; lane L writes 16 L bytes above it
        CHECK(e == tile_dma_elem(i, waves, w, 0) + 8 * lane, "%s: copy destination not M0 + 16 lane", what);
        const uint32_t src = dma_src<D>(swz, e, stride);
        CHECK(src % 16 == 0, "%s: unaligned copy source", what);
        const int el = (int)(src / 2), row = el / stride, col = el % stride;
        CHECK(row == e / D && col + 8 <= D, "%s: copy source (%d, %d) for destination %d", what, row, col, e);
        for (int j = 0; j < 8; ++j) {
          CHECK(tile[e + j].row < 0, "%s: element %d written twice", what, e + j);
          tile[e + j] = Tag{row, col + j};
        }
      }
  std::set<std::pair<int, int>> seen;
  for (const Tag& t : tile) {
    CHECK(t.row >= 0, "%s: element never written", what);
    seen.insert({t.row, t.col});
  }
  CHECK((int)seen.size() == TILE, "%s: the tile does not hold every logical element once", what);
  return tile;
}

// Bank model checks: byte addresses of one read instruction, 64 lanes.
void check_banks_16(const int byte_addr[64], const char* what) {
  for (int g = 0; g < 4; ++g) {
    int used[16] = {0};
    for (int l = 16 * g; l < 16 * g + 16; ++l) ++used[(byte_addr[l] / 16) % 16];
    for (int b = 0; b < 16; ++b) CHECK(used[b] <= 1, "%s: 16-byte reads of lanes %d..%d conflict", what, 16 * g, 16 * g + 15);
  }
}
void check_banks_8(const int byte_addr[64], const char* what) {
  for (int p = 0; p < 2; ++p) {
    int used[32] = {0};
    for (int l = 32 * p; l < 32 * p + 32; ++l) ++used[(byte_addr[l] / 8) % 32];
    for (int b = 0; b < 32; ++b) CHECK(used[b] <= 1, "%s: 8-byte reads of lanes %d..%d conflict", what, 32 * p, 32 * p + 31);
  }
}

// Row fragment (32 rows x 16 columns, 8 per lane) of 32-row block `blk`.
template <int D>
void check_row_frags(const std::vector<Tag>& tile, bool dual, const char* what) {
  constexpr int TILE = 64 * D;
  for (int blk = 0; blk < 2; ++blk)
    for (int t = 0; t < D / 16; ++t) {
      int bytes[64];
      for (int lane = 0; lane < 64; ++lane) bytes[lane] = 2 * ((dual ? row_frag_dual<D>(lane, t) : row_frag_b128<D>(lane, t)) + blk * 32 * D);
      check_banks_16(bytes, what);
      for (int lane = 0; lane < 64; ++lane) {
        const int off = (dual ? row_frag_dual<D>(lane, t) : row_frag_b128<D>(lane, t)) + blk * 32 * D;
        CHECK(off >= 0 && off + 8 <= TILE && off % 8 == 0, "%s: row read %d outside the tile", what, off);
        if (off < 0 || off + 8 > TILE) continue;
        for (int j = 0; j < 8; ++j) {
          const Tag want{32 * blk + perm_rows(lane & 31), 16 * t + 8 * (lane >> 5) + j};
          CHECK(tile[off + j] == want, "%s: lane %d slot %d of row fragment t=%d holds (%d,%d), wants (%d,%d)", what,
                lane, j, t, tile[off + j].row, tile[off + j].col, want.row, want.col);
        }
      }
    }
}

// ds_read_b64_tr_b16: destination lane 16 g + t receives element t % 4 of the
// 4-element units addressed by source lanes 16 g + t / 4 + 4 e, e = 0..3.
void tr16(const std::vector<Tag>& tile, const int addr[64], Tag out[64][4], const char* what) {
  int bytes[64];
  for (int lane = 0; lane < 64; ++lane) {
    CHECK(addr[lane] >= 0 && addr[lane] + 4 <= (int)tile.size() && addr[lane] % 4 == 0,
          "%s: transposing read %d outside the tile", what, addr[lane]);
    bytes[lane] = 2 * addr[lane];
  }
  check_banks_8(bytes, what);
  for (int lane = 0; lane < 64; ++lane) {
    const int g = lane / 16, t = lane % 16;
    for (int e = 0; e < 4; ++e) {
      const int a = addr[16 * g + t / 4 + 4 * e];
      out[lane][e] = (a >= 0 && a + 4 <= (int)tile.size()) ? tile[a + t % 4] : Tag{};
    }
  }
}

// Transposed fragment X^T (32 columns x 16 rows) of column block c and row
// step u: lane l must receive X[16 u + 8 h + j][32 c + l % 32], j = 0..7.
// The forward reads the second half at the first address + 4 D, the
// backward kernels at their own second offset (tr_frag_*(..., 1)).
template <int D>
void check_tr_frags(const std::vector<Tag>& tile, bool dual, bool second_at_plus_4d, const char* what) {
  for (int c = 0; c < D / 32; ++c)
    for (int u = 0; u < 4; ++u) {
      int lo[64], hi[64];
      for (int lane = 0; lane < 64; ++lane) {
        lo[lane] = (dual ? tr_frag_dual<D>(lane, c, 0) : tr_frag_tr<D>(lane, c, 0)) + 16 * u * D;
        hi[lane] = second_at_plus_4d ? lo[lane] + 4 * D
                                     : (dual ? tr_frag_dual<D>(lane, c, 1) : tr_frag_tr<D>(lane, c, 1)) + 16 * u * D;
      }
      Tag a[64][4], b[64][4];
      tr16(tile, lo, a, what);
      tr16(tile, hi, b, what);
      for (int lane = 0; lane < 64; ++lane)
        for (int j = 0; j < 8; ++j) {
          const Tag got = j < 4 ? a[lane][j] : b[lane][j - 4];
          const Tag want{16 * u + 8 * (lane >> 5) + j, 32 * c + (lane & 31)};
          CHECK(got == want, "%s: lane %d slot %d of transposed fragment c=%d u=%d holds (%d,%d), wants (%d,%d)", what,
                lane, j, c, u, got.row, got.col, want.row, want.col);
        }
    }
}

// fp8 tiles: 64 rows x 128 bytes.
std::vector<Tag> fill_fp8_tile(bool is_v, int waves) {
  const int TILE = 64 * 128;
  const int ni = TILE / (waves * 1024);
  const int stride = 3 * 128 + 16;
  std::vector<Tag> tile(TILE);
  for (int w = 0; w < waves; ++w)
    for (int i = 0; i < ni; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int off = fp8_dma_byte(i, waves, w, lane);
        CHECK(off >= 0 && off + 16 <= TILE, "fp8 copy destination %d outside the tile", off);
        if (off < 0 || off + 16 > TILE) continue;
        const uint32_t src = is_v ? fp8_dma_src_v(off, stride) : fp8_dma_src_k(off, stride);
        const int row = (int)(src / stride), col = (int)(src % stride);
        CHECK(row == off / 128 && col % 16 == 0 && col + 16 <= 128, "fp8 copy source (%d, %d)", row, col);
        for (int j = 0; j < 16; ++j) {
          CHECK(tile[off + j].row < 0, "fp8 byte %d written twice", off + j);
          tile[off + j] = Tag{row, col + j};
        }
      }
  for (const Tag& t : tile) CHECK(t.row >= 0, "fp8 byte never written");
  return tile;
}

void check_fp8() {
  for (int waves : {4, 8}) {
    const std::vector<Tag> kt = fill_fp8_tile(false, waves), vt = fill_fp8_tile(true, waves);
    // K row fragments: 32 bytes per lane, k-step t, key block kb
    for (int kb = 0; kb < 2; ++kb)
      for (int t = 0; t < 2; ++t)
        for (int i = 0; i < 2; ++i) {
          int bytes[64];
          for (int lane = 0; lane < 64; ++lane) bytes[lane] = fp8_k_frag(lane, t, i) + kb * 32 * 128;
          check_banks_16(bytes, "fp8 K");
        }
    for (int kb = 0; kb < 2; ++kb)
      for (int t = 0; t < 2; ++t)
        for (int lane = 0; lane < 64; ++lane)
          for (int i = 0; i < 2; ++i) {
            const int off = fp8_k_frag(lane, t, i) + kb * 32 * 128;
            CHECK(off >= 0 && off + 16 <= 64 * 128 && off % 16 == 0, "fp8 K read %d outside the tile", off);
            if (off < 0 || off + 16 > 64 * 128) continue;
            for (int j = 0; j < 16; ++j) {
              const Tag want{32 * kb + perm_rows(lane & 31), 64 * t + 32 * (lane >> 5) + 16 * i + j};
              CHECK(kt[off + j] == want, "fp8 K fragment lane %d byte %d", lane, 16 * i + j);
            }
          }
    // V^T fragments through ds_read_b64_tr_b8: destination lane 16 g + t
    // receives byte t % 8 of the 8-byte segments addressed by source lanes
    // 16 g + t / 8 + 2 e, e = 0..7; byte 8 q + e of lane l must be
    // V[16 q + 8 h + e][32 db + l % 32].
    for (int db = 0; db < 4; ++db)
      for (int q = 0; q < 4; ++q) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          addr[lane] = fp8_v_frag(lane, db) + q * 16 * 128;
          CHECK(addr[lane] >= 0 && addr[lane] + 8 <= 64 * 128 && addr[lane] % 8 == 0, "fp8 V read outside the tile");
        }
        check_banks_8(addr, "fp8 V");
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane / 16, t = lane % 16;
          for (int e = 0; e < 8; ++e) {
            const int a = addr[16 * g + t / 8 + 2 * e];
            const Tag got = (a >= 0 && a + 8 <= 64 * 128) ? vt[a + t % 8] : Tag{};
            const Tag want{16 * q + 8 * (lane >> 5) + e, 32 * db + (lane & 31)};
            CHECK(got == want, "fp8 V^T fragment db=%d q=%d lane %d byte %d holds (%d,%d), wants (%d,%d)", db, q, lane,
                  e, got.row, got.col, want.row, want.col);
          }
        }
      }
  }
}

template <int D>
void check_layouts() {
  char what[96];
  // forward: K (B128 rows) and V (TR, transposed) tiles, 4- and 8-wave workgroups
  for (int waves : {4, 8}) {
    snprintf(what, sizeof what, "fwd D=%d waves=%d K", D, waves);
    check_row_frags<D>(fill_tile<D>(kB128, waves, what), false, what);
    snprintf(what, sizeof what, "fwd D=%d waves=%d V", D, waves);
    check_tr_frags<D>(fill_tile<D>(kTR, waves, what), false, true, what);
  }
  // dK/dV: Q and dO tiles (dual: rows for S and dP, transposed for dV and dK), 8 waves
  snprintf(what, sizeof what, "dkdv D=%d Q/dO", D);
  {
    const std::vector<Tag> t = fill_tile<D>(kDual, 8, what);
    check_row_frags<D>(t, true, what);
    check_tr_frags<D>(t, true, false, what);
  }
  // dQ: K tile dual (rows for S, transposed for dQ), V tile B128 rows, 4 or 8 waves
  for (int waves : {4, 8}) {
    snprintf(what, sizeof what, "dq D=%d waves=%d K", D, waves);
    {
      const std::vector<Tag> t = fill_tile<D>(kDual, waves, what);
      check_row_frags<D>(t, true, what);
      check_tr_frags<D>(t, true, false, what);
    }
    snprintf(what, sizeof what, "dq D=%d waves=%d V", D, waves);
    check_row_frags<D>(fill_tile<D>(kB128, waves, what), false, what);
  }
}

// ---------------------------------------------------------------------------
// Tile ranges of query blocks (forward, dQ) and key blocks (dK/dV).
// ---------------------------------------------------------------------------
struct Shape {
  int seqlen;
  bool causal;
  std::vector<int32_t> cu;  // empty: one dense sequence
};

void visible_keys(const Shape& s, int q, int& lo, int& hi) {
  int s0, s1;
  segment_of(s.cu.empty() ? nullptr : s.cu.data(), (int)s.cu.size() - 1, s.seqlen, q, s0, s1);
  lo = s0;
  hi = s.causal ? q + 1 : s1;
}

void check_ranges(const Shape& s) {
  const int S = s.seqlen, ntiles = (S + 63) / 64;
  // forward and dQ: block of BM queries, visible keys [min lo, max hi) -> tiles
  for (int bm : {128, 256}) {
    for (int blk = 0; blk * bm < S; ++blk) {
      int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
      for (int q = blk * bm; q < imin(S, (blk + 1) * bm); ++q) {
        int lo, hi;
        visible_keys(s, q, lo, hi);
        CHECK(0 <= lo && lo <= q && q < hi && hi <= S, "row %d visible range [%d, %d)", q, lo, hi);
        wg_lo = imin(wg_lo, lo);
        wg_hi = imax(wg_hi, hi);
      }
      const int tb = wg_hi > wg_lo ? wg_lo / 64 : 0;
      const int te = wg_hi > wg_lo ? (wg_hi + 63) / 64 : 0;
      CHECK(0 <= tb && tb <= te && te <= ntiles, "block %d tiles [%d, %d) of %d", blk, tb, te, ntiles);
      for (int q = blk * bm; q < imin(S, (blk + 1) * bm); ++q) {
        int lo, hi;
        visible_keys(s, q, lo, hi);
        CHECK(tb * 64 <= lo && hi <= te * 64, "row %d keys [%d, %d) outside its block's tiles", q, lo, hi);
      }
      // key-split shares of the tiles: disjoint, in order, covering
      for (int ks : {1, 2, 3, 4, 8}) {
        int prev = tb;
        for (int sh = 0; sh < ks; ++sh) {
          int a, b;
          share_range(te - tb, ks, sh, a, b);
          CHECK(tb + a == prev && a <= b, "share %d of %d of tiles [%d, %d)", sh, ks, tb, te);
          prev = tb + b;
        }
        CHECK(prev == te, "shares of %d do not cover [%d, %d)", ks, tb, te);
      }
    }
  }
  // dK/dV: block of 128 keys, the queries that see them -> 64-query tiles
  for (int blk = 0; blk * 128 < S; ++blk) {
    int wg_lo = INT32_MAX, wg_hi = INT32_MIN;
    for (int k = blk * 128; k < imin(S, (blk + 1) * 128); ++k) {
      int s0, s1;
      segment_of(s.cu.empty() ? nullptr : s.cu.data(), (int)s.cu.size() - 1, S, k, s0, s1);
      const int qlo = s.causal ? k : s0, qhi = s1;
      wg_lo = imin(wg_lo, qlo);
      wg_hi = imax(wg_hi, qhi);
    }
    const int tb = wg_hi > wg_lo ? wg_lo / 64 : 0, te = wg_hi > wg_lo ? (wg_hi + 63) / 64 : 0;
    CHECK(0 <= tb && tb <= te && te <= ntiles, "key block %d query tiles [%d, %d)", blk, tb, te);
    for (int k = blk * 128; k < imin(S, (blk + 1) * 128); ++k) {
      int s0, s1;
      segment_of(s.cu.empty() ? nullptr : s.cu.data(), (int)s.cu.size() - 1, S, k, s0, s1);
      const int qlo = s.causal ? k : s0;
      CHECK(tb * 64 <= qlo && s1 <= te * 64, "key %d queries [%d, %d) outside its block's tiles", k, qlo, s1);
    }
  }
}

// ---------------------------------------------------------------------------
// Workspace layouts and 32-bit copy ranges
// ---------------------------------------------------------------------------
void check_workspace(int B, int Hq, int Hkv, int S, int D) {
  const int hs = bwd_head_split(B, Hq, Hkv, S), ks = bwd_key_split(B, Hq, S);
  CHECK(hs >= 1 && hs <= Hq / Hkv && ks >= 1 && ks <= 4, "splits %d %d", hs, ks);
  const size_t stat = (size_t)4 * B * Hq * stat_stride_for(S);
  const size_t nblk = ((size_t)S + 127) / 128;
  const size_t order = bwd_order_offset(B, Hq, S);
  CHECK(order == 2 * stat, "order offset");
  const size_t part = bwd_part_offset(B, Hq, S, hs, ks);
  CHECK(part % 256 == 0 && part >= order + 4 * nblk * (hs + ks), "partial dK/dV offset");
  const size_t dqp = bwd_dq_part_offset(B, Hq, Hkv, S, D, hs, ks);
  const size_t part_bytes = hs > 1 ? (size_t)8 * hs * B * S * Hkv * D : 0;
  CHECK(dqp % 256 == 0 && dqp >= part + part_bytes, "partial dQ offset");
  const size_t total = bwd_workspace_size(B, Hq, Hkv, S, D);
  const size_t dq_bytes = ks > 1 ? (size_t)4 * ks * B * S * Hq * D : 0;
  CHECK(total == dqp + dq_bytes, "workspace size");
  const int fks = fwd_key_split(B, Hq, S);
  CHECK(fks >= 1 && fks <= kFwdMaxKeySplit, "forward split %d", fks);
  if (fks > 1) {
    CHECK(((S + 63) / 64) / fks >= kFwdMinTilesPerShare - 1, "forward share too short");
    const size_t lse_off = fwd_part_lse_offset(B, Hq, S, D, fks);
    CHECK(lse_off % 256 == 0 && lse_off >= (size_t)4 * fks * B * S * Hq * D, "forward workspace offsets");
    CHECK(fwd_workspace_size(B, Hq, S, D) == lse_off + (size_t)4 * fks * B * Hq * S, "forward workspace size");
  } else {
    CHECK(fwd_workspace_size(B, Hq, S, D) == 0, "unsplit forward needs no workspace");
  }
  // tile copies address one batch slice's rows with 32-bit byte ranges:
  // (S - t0) * stride * 2 for the tile starting at t0 must fit, stride = H * D
  const uint64_t kv_bytes = (uint64_t)S * Hkv * D * 2, q_bytes = (uint64_t)S * Hq * D * 2;
  CHECK(kv_bytes <= UINT32_MAX && q_bytes <= UINT32_MAX, "copy byte range of S=%d Hq=%d D=%d exceeds 32 bits", S, Hq, D);
  CHECK((uint64_t)S * Hq * D <= (uint64_t)INT32_MAX, "element offsets of S=%d Hq=%d D=%d exceed 31 bits", S, Hq, D);
}

// The debug build's LDS access rule (lds_access_ok): inside the allocation,
// aligned, and no wrap-around at the top of the 32-bit address range.
void check_lds_rule() {
  CHECK(lds_access_ok(0, 16, 16, 16), "lds rule: whole allocation");
  CHECK(lds_access_ok(48, 16, 16, 64), "lds rule: last chunk");
  CHECK(!lds_access_ok(64, 16, 16, 64), "lds rule: one past the end");
  CHECK(!lds_access_ok(56, 16, 16, 64), "lds rule: straddles the end (and misaligned)");
  CHECK(!lds_access_ok(8, 16, 16, 64), "lds rule: misaligned 16-byte access");
  CHECK(lds_access_ok(8, 8, 8, 64), "lds rule: aligned 8-byte access");
  CHECK(!lds_access_ok(4, 8, 8, 64), "lds rule: misaligned 8-byte access");
  CHECK(!lds_access_ok(0xFFFFFFF0u, 16, 16, 64), "lds rule: address beyond the allocation");
  CHECK(!lds_access_ok(0xFFFFFFF0u, 32, 16, 0xFFFFFFF8u), "lds rule: wrap-around");
  CHECK(lds_access_ok(160 * 1024 - 16, 16, 16, 160 * 1024), "lds rule: top of a 160 KB allocation");
  CHECK(!lds_access_ok(0, 16, 16, 0), "lds rule: empty allocation");
}

// The rows of the one-wave-per-row kernels (the forward's few-key rows and
// the backward's Delta from its definition): for every segment length and
// mask, row r of the segment is one of rows [0, few_key_rows) exactly when it
// sees fewer than 64 keys, the grid's 4-row blocks cover those rows, and the
// keys a row reads and the staged K/V rows stay inside the 63-row LDS arrays.
void check_few_key_rows() {
  constexpr int kBlocks = 16, kRowsPerWg = 4, kLdsRows = kFewKeyLimit - 1;
  for (int len = 0; len <= 300; ++len)
    for (bool causal : {true, false}) {
      const int n = few_key_rows(len, causal);
      CHECK(0 <= n && n <= len && n <= kLdsRows, "few-key rows: len %d causal %d gives %d rows", len, causal, n);
      CHECK(n <= kBlocks * kRowsPerWg, "few-key rows: %d rows, %d blocks of %d", n, kBlocks, kRowsPerWg);
      for (int r = 0; r < len; ++r) {
        const int visible = causal ? r + 1 : len;
        CHECK((visible < kFewKeyLimit) == (r < n), "few-key rows: len %d causal %d row %d sees %d keys", len, causal,
              r, visible);
        if (r < n) CHECK(visible <= n, "few-key rows: row %d reads %d keys of %d staged", r, visible, n);
      }
    }
  // the bank swizzle (c + j) % C of the staged rows is a permutation of each row's chunks
  for (int C : {8, 16})
    for (int j = 0; j < kLdsRows; ++j) {
      std::set<int> seen;
      for (int c = 0; c < C; ++c) seen.insert((c + j) % C);
      CHECK((int)seen.size() == C, "few-key rows: swizzle of row %d", j);
    }
}

int main() {
  check_lds_rule();
  check_few_key_rows();
  check_layouts<128>();
  check_layouts<64>();
  check_fp8();

  // sequence shapes: dense causal / non-causal, ragged tails, packed lengths
  std::vector<Shape> shapes;
  for (int S : {1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4096, 4097})
    for (bool c : {true, false}) shapes.push_back(Shape{S, c, {}});
  const std::vector<std::vector<int>> packs = {
      {1}, {1, 1, 1}, {5, 1, 14}, {64, 64, 128, 64}, {100, 1, 1, 64, 65, 500, 269}, {300, 400}, {1, 16, 239},
      {6091, 7755, 7282, 4439, 7201}, {4000, 500}, {63, 1, 64, 127, 129}};
  for (const auto& lens : packs)
    for (bool c : {true, false}) {
      Shape s{0, c, {0}};
      for (int L : lens) {
        s.seqlen += L;
        s.cu.push_back(s.seqlen);
      }
      shapes.push_back(s);
    }
  unsigned rng = 12345;
  for (int r = 0; r < 40; ++r) {  // seeded random packings
    Shape s{0, (r & 1) == 0, {0}};
    const int n = 1 + (int)((rng = rng * 1103515245u + 12345u) >> 16) % 12;
    for (int i = 0; i < n; ++i) {
      const int L = 1 + (int)((rng = rng * 1103515245u + 12345u) >> 16) % 700;
      s.seqlen += L;
      s.cu.push_back(s.seqlen);
    }
    shapes.push_back(s);
  }
  for (const Shape& s : shapes) check_ranges(s);
  // malformed prefix sums (not checked on the device by default): every row's
  // range must still lie inside the sequence, so no access leaves the tensors
  const std::vector<std::pair<int, std::vector<int32_t>>> bad = {
      {256, {0, 300}}, {256, {0, 100, 50, 256}}, {256, {-5, 10, 256}}, {256, {0, 100, 100, 256}},
      {200, {0, 50, 500, 100}}, {64, {10, 20}}, {300, {0, 7, 7, 7, 400}}};
  for (const auto& b : bad)
    for (bool c : {true, false}) {
      Shape s{b.first, c, b.second};
      for (int q = 0; q < s.seqlen; ++q) {
        int lo, hi;
        visible_keys(s, q, lo, hi);
        CHECK(0 <= lo && lo <= q && q < hi && hi <= s.seqlen, "malformed cu: row %d range [%d, %d) of %d", q, lo, hi,
              s.seqlen);
      }
    }

  // workspace layouts over a size sweep, up to the largest accepted sequence
  for (int D : {64, 128})
    for (int Hkv : {1, 2, 4})
      for (int G : {1, 2, 3, 7, 8})
        for (int B : {1, 2, 3})
          for (int S : {1, 5, 64, 65, 129, 1000, 4032, 4033, 8192, 32768, 262144}) check_workspace(B, Hkv * G, Hkv, S, D);
  for (int D : {64, 128})
    for (int Hq : {1, 2, 7, 28, 32}) {
      const int S = (int)(((uint64_t)INT32_MAX) / ((uint64_t)Hq * D));  // seqlen * Hq * D <= 2^31 - 1
      for (int Hkv : {1, Hq}) check_workspace(1, Hq, Hkv, S, D);
    }

  printf("index_check: %ld checks, %d failures\n", g_checks, g_fail);
  if (g_fail) return 1;
  printf("index_check: OK\n");
  return 0;
}
