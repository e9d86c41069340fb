// Transposable 2:4 mask search and 2:4 compression kernels for gfx950.
//
// Method: "Accelerating Transformer Pre-training with 2:4 Sparsity",
// Algorithm 1 (transposable mask search: |W|, a stride-4 correlation with the
// 90 transposable patterns, argmax over patterns) and the pruning kernel of
// the "Software Dependencies" row of its reproducibility table.  The pages
// give the correlation as a conv2d; here it is a per-block search in
// registers: the score tensor is never materialised.
//
// Score semantics (fixed by the library): a pattern's score is the fp32 sum of
// the 8 kept magnitudes added in row-major order from +0, and the first
// maximum in pattern order wins.  Two code paths compute exactly that:
//
//  * search_fast, for blocks whose sums are all exact in fp32.  With e the
//    fp16 exponent field, a block is exact when emax - max(emin_nonzero, 1)
//    <= 10: every entry is then an integer multiple of q = 2^(emin-25) below
//    2^21 q, so every sum of up to 8 entries is an integer multiple of q below
//    2^24 q and is exact in fp32 whatever the order of additions.  The sums are
//    then formed as integers in units of q, shifted left by 7, with 127 - index
//    in the low 7 bits, so an unsigned max returns the highest score and, among
//    equal scores, the lowest index.  The score splits into rows 0-1 ("top")
//    and rows 2-3 ("bottom"); the column counts of the top pair fix which
//    bottom pairs complete it (19 deficit classes), so the best pattern is the
//    max over classes of (best top key + best bottom key).
//  * search_exact_order, for every other block (and Inf/NaN): the 90
//    sequential fp32 sums in row-major order with a strict > scan.
//
// Compression layouts: see include/sp24.h.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>
#include <utility>

#include "sp24_device.hpp"
#include "sp24_internal.hpp"
#include "sp24_patterns.hpp"

namespace sp24 {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}
__device__ __forceinline__ uint32_t pk_m_inu16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}
__device__ __forceinline__ uint32_t pk_dec_u16(uint32_t a) {
  // subtract 1 from each 16-bit half, wrapping (0 -> 0xFFFF)
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(us2, a) - us2{1, 1});
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// m[r][h]: sign-cleared fp16 pairs of block row r; h = 0 holds columns 0 (low
// half) and 1, h = 1 holds columns 2 and 3.
struct BlockMag {
  uint32_t m[4][2];
};

// Exponent range of the block: returns true (fast path usable) and the scale
// exponent emin' when all partial sums are exact in fp32.
__device__ __forceinline__ bool exact_regime(const BlockMag& b, int& em_inout) {
  uint32_t mx = pk_max_u16(pk_max_u16(pk_max_u16(b.m[0][0], b.m[0][1]), pk_max_u16(b.m[1][0], b.m[1][1])),
                           pk_max_u16(pk_max_u16(b.m[2][0], b.m[2][1]), pk_max_u16(b.m[3][0], b.m[3][1])));
  uint32_t mn = pk_m_inu16(pk_m_inu16(pk_m_inu16(pk_dec_u16(b.m[0][0]), pk_dec_u16(b.m[0][1])),
                                      pk_m_inu16(pk_dec_u16(b.m[1][0]), pk_dec_u16(b.m[1][1]))),
                           pk_m_inu16(pk_m_inu16(pk_dec_u16(b.m[2][0]), pk_dec_u16(b.m[2][1])),
                                      pk_m_inu16(pk_dec_u16(b.m[3][0]), pk_dec_u16(b.m[3][1]))));
  const uint32_t hmax = max(mx & 0xFFFFu, mx >> 16);
  const uint32_t hm_innz = min(mn & 0xFFFFu, mn >> 16) + 1u;  // 0x10000 when all entries are zero
  const int emax = (int)(hmax >> 10);
  const int emin = max((int)(hm_innz >> 10), 1);                 // 64 when all entries are zero
  em_inout = emin;
  return emax < 31 && emax - emin <= 10;
}

// Tie-break offsets of the keys, moved between the two halves of a class.
// A top key carries 122 - top_base and a bottom key 5 - bot_rank, whose sum
// over a class's top and bottom is 127 - index.  Taking K_c from every top
// constant of class c and giving it to every bottom constant of that class
// leaves each sum unchanged, and brings the constants into 0..64: operands
// that a three-input add takes inline, where larger ones cost a second
// instruction.  None is negative, so a key of a zero score cannot wrap.
struct KeyOffsets {
  uint32_t top[36], bot[36];
};
constexpr KeyOffsets build_key_offsets() {
  KeyOffsets o{};
  int shift[kNumClasses] = {};
  for (int c = 0; c < kNumClasses; ++c) {
    int lo = 1 << 20, hi = -1;
    for (int p = 0; p < 36; ++p)
      if (kTables.pair_class[p] == c) {
        const int ct = 122 - kTables.top_base[p];
        lo = ct < lo ? ct : lo;
        hi = ct > hi ? ct : hi;
      }
    int k = hi - 64 > 0 ? hi - 64 : 0;   // every top constant at most 64 ...
    k = k < lo ? k : lo;                  // ... unless that needs one below 0
    shift[c] = k < 59 ? k : 59;           // bottom constants (at most 5 + k) at most 64
  }
  for (int p = 0; p < 36; ++p) {
    o.top[p] = (uint32_t)(122 - kTables.top_base[p] - shift[kTables.pair_class[p]]);
    o.bot[p] = (uint32_t)(5 - kTables.bot_rank[p] + shift[kTables.bot_class[p]]);
  }
  return o;
}
constexpr KeyOffsets kKeyOff = build_key_offsets();
constexpr bool key_offsets_ok() {
  bool ok = true;
  for (int p = 0; p < 36; ++p) ok = ok && (int)kKeyOff.top[p] >= 0 && kKeyOff.top[p] < 128 && kKeyOff.bot[p] <= 64;
  // every pattern's two offsets still sum to 127 - index
  for (int i = 0; i < kNumPatterns; ++i) {
    const int tp = 6 * kTables.code[i][0] + kTables.code[i][1];
    const int bp = 6 * kTables.code[i][2] + kTables.code[i][3];
    ok = ok && kKeyOff.top[tp] + kKeyOff.bot[bp] == (uint32_t)(127 - i);
  }
  return ok;
}
static_assert(key_offsets_ok(), "key offsets");

// a + b + C as one instruction when C is an inline constant (0..64); the
// compiler would share a + C between keys that have the same C, at three
// instructions for two keys
template <uint32_t C>
__device__ __forceinline__ uint32_t add3_const(uint32_t a, uint32_t b) {
  if constexpr (C <= 64) {
    uint32_t r;
    asm("v_add3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "n"(C));
    return r;
  } else {
    return a + b + C;
  }
}

__device__ __forceinline__ int search_fast(const BlockMag& b, int emin) {
  // scale 2^(25 - emin): entries become integers below 2^21.  fma(x, s, 2^23)
  // is exact and its bit pattern is 0x4B000000 + integer.
  const float scale = __uint_as_float((uint32_t)(25 - emin + 127) << 23);
  uint32_t q[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    q[r][0] = __float_as_uint(__builtin_fmaf(half_lo(b.m[r][0]), scale, 8388608.0f));
    q[r][1] = __float_as_uint(__builtin_fmaf(half_hi(b.m[r][0]), scale, 8388608.0f));
    q[r][2] = __float_as_uint(__builtin_fmaf(half_lo(b.m[r][1]), scale, 8388608.0f));
    q[r][3] = __float_as_uint(__builtin_fmaf(half_hi(b.m[r][1]), scale, 8388608.0f));
  }
  // Pair sums shifted left by 7.  The two 0x4B000000 offsets sum to
  // 0x96000000, which vanishes modulo 2^32 after the shift.
  // The shift is opaque to the compiler: knowing the low 7 bits zero, it
  // turns the key offset additions below into ORs, which a three-input add
  // cannot absorb.
  uint32_t P[4][6];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int k = 0; k < 6; ++k)
      asm("v_add_lshl_u32 %0, %1, %2, 7" : "=v"(P[r][k]) : "v"(q[r][kPairLo[k]]), "v"(q[r][kPairHi[k]]));
  // best top and bottom key per deficit class
  uint32_t top[kNumClasses], bot[kNumClasses];
  bool top_set[kNumClasses] = {}, bot_set[kNumClasses] = {};
  [&]<int... ps>(std::integer_sequence<int, ps...>) {
    ([&] {
      constexpr int p = ps, x = p / 6, y = p % 6;
      const uint32_t tk = add3_const<kKeyOff.top[p]>(P[0][x], P[1][y]);
      const uint32_t bk = add3_const<kKeyOff.bot[p]>(P[2][x], P[3][y]);
      constexpr int tc = kTables.pair_class[p], bc = kTables.bot_class[p];
      top[tc] = top_set[tc] ? max(top[tc], tk) : tk;
      top_set[tc] = true;
      bot[bc] = bot_set[bc] ? max(bot[bc], bk) : bk;
      bot_set[bc] = true;
    }(), ...);
  }(std::make_integer_sequence<int, 36>{});
  uint32_t best = top[0] + bot[0];
#pragma unroll
  for (int k = 1; k < kNumClasses; ++k) best = max(best, top[k] + bot[k]);
  return 127 - (int)(best & 127u);
}

// Out of line: only blocks outside the exact regime take it.  The block is
// passed by value, in registers: a reference would make every caller store
// the block to scratch memory, taken or not.
__device__ __noinline__ int search_exact_order(BlockMag b) {
  constexpr const PatternTables& T = kTables;
  float a[16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a[4 * r + 0] = half_lo(b.m[r][0]);
    a[4 * r + 1] = half_hi(b.m[r][0]);
    a[4 * r + 2] = half_lo(b.m[r][1]);
    a[4 * r + 3] = half_hi(b.m[r][1]);
  }
  float best_s = 0.0f;
  int best = 0;
#pragma unroll
  for (int p = 0; p < kNumPatterns; ++p) {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (T.mask[p] & (1u << e)) s = s + a[e];
    if (p == 0) {
      best_s = s;
    } else if (s > best_s) {
      best_s = s;
      best = p;
    }
  }
  return best;
}

__device__ __forceinline__ int search_block(const BlockMag& b) {
  int emin;
  if (exact_regime(b, emin)) return search_fast(b, emin);
  return search_exact_order(b);
}

__device__ __forceinline__ BlockMag load_block(const uint32_t (&w)[4][2]) {
  BlockMag b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    b.m[r][0] = w[r][0] & 0x7FFF7FFFu;
    b.m[r][1] = w[r][1] & 0x7FFF7FFFu;
  }
  return b;
}

// ---------------------------------------------------------------------------
// mask search only

constexpr int kSearchThreads = 256;

__global__ __launch_bounds__(kSearchThreads) void mask_search_kernel(const uint16_t* __restrict__ W, int64_t R,
                                                                     int64_t C, uint8_t* __restrict__ idx) {
  const int64_t nbc = C / 4;
  const int64_t nblocks = (R / 4) * nbc;
  for (int64_t blk = (int64_t)blockIdx.x * kSearchThreads + threadIdx.x; blk < nblocks;
       blk += (int64_t)gridDim.x * kSearchThreads) {
    const int64_t bi = blk / nbc, bj = blk - bi * nbc;
    uint32_t w[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint2 v = *reinterpret_cast<const uint2*>(W + (4 * bi + r) * C + 4 * bj);
      w[r][0] = v.x;
      w[r][1] = v.y;
    }
    idx[blk] = (uint8_t)search_block(load_block(w));
  }
}

// ---------------------------------------------------------------------------
// search (or read idx) + compress, one 128x128 tile of one weight per
// workgroup; one launch may cover several weights (a job table)

constexpr int kTile = 128;            // rows and columns of W per workgroup
constexpr int kTB = kTile / 4;        // blocks per tile side (32)
constexpr int kCompressThreads = 256;
constexpr int kBlocksPerThread = kTB * kTB / kCompressThreads;  // 4
constexpr int kCompressWaves = kCompressThreads / 64;
// Each workgroup handles kTilesPerWg tiles (see search_compress_kernel).
// One is fastest at the 1.5B shapes (both weights from HBM: 46.2 us against
// 50.2 us with two; cache-resident: 29.6 us against 34.8 us with two and
// 38.7 us with three): with about three workgroups resident per
// CU, later workgroups start as earlier ones finish, so loads, searches and
// stores of different tiles overlap on each CU.  Smaller 64 x 64 tiles are
// slower (44-68 us): each workgroup adds its flip count with one same-address
// atomic, and those serialise.
constexpr int kTilesPerWg = 1;

// v_perm_b32 byte selector that gathers halves i0 and i1 of a 4-half group
// held in two dwords (bytes 2*i0, 2*i0+1, 2*i1, 2*i1+1), from the nibble
// i0 | i1 << 2.  Computed in a few VALU operations rather than looked up:
// per-lane lookups of a per-pattern table land on a quarter of the LDS banks.
__device__ __forceinline__ uint32_t pair_selector(uint32_t nib) {
  // i0 into byte 0 and i1 into byte 2; one 24-bit multiply-add by 0x202 then
  // doubles each and copies it into the byte above (no carries: i < 4)
  const uint32_t spread = (nib & 3u) | (nib >> 2) << 16;
  return spread * 0x0202u + 0x01000100u;
}

// One 8-byte entry per pattern: x = row nibbles (bits 0..15) | column
// nibbles << 16, y = kept entries (bit 4r+c).
struct PatTable {
  uint2 entry[kNumPatterns];
};

constexpr PatTable build_pat_table() {
  PatTable t{};
  for (int p = 0; p < kNumPatterns; ++p) {
    t.entry[p].x = (uint32_t)kTables.row_nib[p] | (uint32_t)kTables.col_nib[p] << 16;
    t.entry[p].y = kTables.mask[p];
  }
  return t;
}

__constant__ PatTable g_pat = build_pat_table();

// The column form is staged with the row-group index of columns 64 .. 127 of
// the tile XOR 1, so that the 32 lanes storing one row group of 32 block
// columns (stride 4 rows of 33 dwords) cover 32 distinct banks.
__device__ __forceinline__ int col_swz(int column) { return (column >> 6) & 1; }

struct CompressSmem {
  PatTable pat;
  uint32_t vals_row[kTile][kTB + 1];     // [row][group]: kept pair as one dword
  uint32_t vals_col[kTile][kTB + 1];     // [column][row group ^ col_swz(column)]
  uint32_t bnibs[kTB][kTB + 1];          // [block row][block column]: nibbles of the block's pattern
  uint8_t idx[kTB][kTB];
  uint8_t prev[kTilesPerWg][kTB][kTB];          // previous indices of each tile (flip counting)
  uint32_t flips[kTilesPerWg][kCompressWaves];  // per-wave flip counts of each tile
};
static_assert(sizeof(PatTable) % 4 == 0, "the pattern table is copied in dwords");
static_assert(kCompressThreads == 256 && kTile == 128, "write_full_tile: 8 lanes per 128-byte row, 32 rows per pass");

// Tile geometry of one workgroup-tile of one job.  The job is copied by
// value (selected with static indices), so the kernel-argument table never
// needs an address and stays in scalar registers.
struct TileRef {
  ScJob jb;
  int64_t r0, c0;
  int rows, cols;
};

__device__ __forceinline__ TileRef tile_ref(const ScJobs& jobs, int64_t t) {
  ScJob jb = jobs.j[0];
#pragma unroll
  for (int k = 1; k < kMaxScJobs; ++k)
    if (k < jobs.count && t >= jobs.j[k].tile_begin) jb = jobs.j[k];
  const int64_t u = t - jb.tile_begin;
  const int64_t ti = u / jb.tiles_c, tj = u - ti * jb.tiles_c;
  TileRef tr;
  tr.jb = jb;
  tr.r0 = ti * kTile;
  tr.c0 = tj * kTile;
  tr.rows = (int)min<int64_t>(kTile, jb.R - tr.r0);
  tr.cols = (int)min<int64_t>(kTile, jb.C - tr.c0);
  return tr;
}

// This thread's four blocks of one tile: rows 4*bi .. 4*bi+3 of block row
// bi = tid/32 + 8q, columns 4*bj .. 4*bj+3.
struct TileData {
  uint32_t w[kBlocksPerThread][4][2];
  uint32_t prev4;   // four previous indices: block row tid/8, block columns 4*(tid%8) .. +3
};

// Previous indices of a tile, one dword (four blocks) per thread.  The loads
// here and in load_tile are branch-free (indices past a partial tile are
// clamped to its last block and the values never used), so the compiler can
// count them exactly and wait for just the ones it needs.
__device__ __forceinline__ void load_prev(const TileRef& tr, int tid, TileData& d) {
  const int bi = min(tid / 8, tr.rows / 4 - 1), bj4 = min(4 * (tid % 8), tr.cols / 4 - 4);
  d.prev4 = *reinterpret_cast<const uint32_t*>(tr.jb.idx_prev + (tr.r0 / 4 + bi) * (tr.jb.C / 4) + tr.c0 / 4 + bj4);
}

__device__ __forceinline__ void load_tile(const TileRef& tr, int tid, TileData& d) {
  const int bj = min(tid % kTB, tr.cols / 4 - 1);
#pragma unroll
  for (int q = 0; q < kBlocksPerThread; ++q) {
    const int bi = min(tid / kTB + q * (kCompressThreads / kTB), tr.rows / 4 - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint2 v = *reinterpret_cast<const uint2*>(tr.jb.W + (tr.r0 + 4 * bi + r) * tr.jb.C + tr.c0 + 4 * bj);
      d.w[q][r][0] = v.x;
      d.w[q][r][1] = v.y;
    }
  }
}

// Search (or read the given masks), then stage both compressed forms of the
// tile in LDS.  Returns this thread's count of mask entries that changed
// against the previous masks (0 unless the job counts flips).
template <bool kSearch>
__device__ __forceinline__ uint32_t stage_tile(const TileRef& tr, int k, int tid, const TileData& d,
                                               CompressSmem& sm) {
  const ScJob& jb = tr.jb;
  const int bj = tid % kTB;
  const int nbc_t = tr.cols / 4, nbr_t = tr.rows / 4;
  uint32_t flips = 0;
#pragma unroll
  for (int q = 0; q < kBlocksPerThread; ++q) {
    const int bi = tid / kTB + q * (kCompressThreads / kTB);
    if (bi >= nbr_t || bj >= nbc_t) continue;
    const uint32_t(&w)[4][2] = d.w[q];
    int p;
    if constexpr (kSearch) {
      p = search_block(load_block(w));
    } else {
      p = jb.idx_in[(tr.r0 / 4 + bi) * (jb.C / 4) + tr.c0 / 4 + bj];
      p = p < kNumPatterns ? p : 0;
    }
    sm.idx[bi][bj] = (uint8_t)p;
    const uint2 ent = sm.pat.entry[p];
    if (kSearch && jb.idx_prev) {
      const uint32_t pv = sm.prev[k][bi][bj];
      const uint32_t prev = pv < (uint32_t)kNumPatterns ? pv : 0u;
      flips += (uint32_t)__builtin_popcount(ent.y ^ sm.pat.entry[prev].y);
    }
    const uint32_t nibs = ent.x;
    sm.bnibs[bi][bj] = nibs;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.vals_row[4 * bi + r][bj] = __builtin_amdgcn_perm(w[r][1], w[r][0], pair_selector((nibs >> (4 * r)) & 0xF));
    const int cs = col_swz(4 * bj);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t hsel = (c & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t top = __builtin_amdgcn_perm(w[1][c >> 1], w[0][c >> 1], hsel);  // rows 0,1 of column c
      const uint32_t bot = __builtin_amdgcn_perm(w[3][c >> 1], w[2][c >> 1], hsel);  // rows 2,3
      sm.vals_col[4 * bj + c][bi ^ cs] = __builtin_amdgcn_perm(bot, top, pair_selector((nibs >> (16 + 4 * c)) & 0xF));
    }
  }
  return flips;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// Stores of a whole 128 x 128 tile (every tile but those on a weight's ragged
// edge).  Lane tid writes 16-byte segment tid % 8 of rows (and columns)
// tid / 8 + 32 k, so its addresses are computed once and then advance by a
// uniform stride: no per-segment division or 64-bit multiply.  In the forms'
// blocked order the tile covers two 64-row bands and two column blocks, all
// full: pass k writes rows 32k .. 32k+31, in band k / 2 at row 32 (k % 2) of
// the band, and each wave's 8 rows of a block are 512 contiguous bytes.
__device__ __forceinline__ void write_full_tile(const TileRef& tr, int tid, const CompressSmem& sm) {
  const ScJob& jb = tr.jb;
  const int64_t R = jb.R, C = jb.C, r0 = tr.r0, c0 = tr.c0;
  constexpr int kStep = kCompressThreads / 8;   // rows (columns) per pass: 32
  const int g4 = tid % 8, r = tid / 8;
  if (jb.idx_out) {
    // block row r, blocks 4*g4 .. 4*g4+3
    const uint32_t v = (uint32_t)sm.idx[r][4 * g4] | (uint32_t)sm.idx[r][4 * g4 + 1] << 8 |
                       (uint32_t)sm.idx[r][4 * g4 + 2] << 16 | (uint32_t)sm.idx[r][4 * g4 + 3] << 24;
    *reinterpret_cast<uint32_t*>(jb.idx_out + (r0 / 4 + r) * (C / 4) + c0 / 4 + 4 * g4) = v;
  }
  // offsets within a band: column block g4 / 4, row r, segment (word) g4 % 4
  const int vin = (g4 / 4) * 64 * (int)kValsBlock + r * (int)kValsBlock + 8 * (g4 % 4);
  const int m_in = (g4 / 4) * 64 * (int)kMetaBlock + r * (int)kMetaBlock + (g4 % 4);
  if (jb.vals_row) {
    // bands of 64 rows of C/2 halves (C/16 words); the tile's first column
    // block starts at half c0/2 (word c0/16) of the band's columns
    uint16_t* vp = jb.vals_row + r0 * (C / 2) + (c0 / 2) * 64 + vin;
    uint16_t* mp = jb.meta_row + r0 * (C / 16) + (c0 / 16) * 64 + m_in;
    const int64_t vband = 64 * (C / 2), mband = 64 * (C / 16);
    const int sh = 4 * (r & 3);   // the row within its block (kStep is a multiple of 4)
#pragma unroll
    for (int k = 0; k < kTile / kStep; ++k) {
      const int rr = r + kStep * k;
      const int64_t vo = (k / 2) * vband + (k % 2) * kStep * kValsBlock;
      const int64_t mo = (k / 2) * mband + (k % 2) * kStep * kMetaBlock;
      *reinterpret_cast<uint4*>(vp + vo) =
          make_uint4(sm.vals_row[rr][4 * g4 + 0], sm.vals_row[rr][4 * g4 + 1], sm.vals_row[rr][4 * g4 + 2],
                     sm.vals_row[rr][4 * g4 + 3]);
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) word |= ((sm.bnibs[rr >> 2][4 * g4 + q] >> sh) & 0xFu) << (4 * q);
      mp[mo] = (uint16_t)word;
    }
  }
  if (jb.vals_col) {
    uint16_t* vp = jb.vals_col + c0 * (R / 2) + (r0 / 2) * 64 + vin;
    uint16_t* mp = jb.meta_col + c0 * (R / 16) + (r0 / 16) * 64 + m_in;
    const int64_t vband = 64 * (R / 2), mband = 64 * (R / 16);
    const int sh = 16 + 4 * (r & 3);
#pragma unroll
    for (int k = 0; k < kTile / kStep; ++k) {
      const int c = r + kStep * k;
      const int cs = col_swz(kStep * k);   // equals col_swz(c), since r < kStep
      const int64_t vo = (k / 2) * vband + (k % 2) * kStep * kValsBlock;
      const int64_t mo = (k / 2) * mband + (k % 2) * kStep * kMetaBlock;
      *reinterpret_cast<uint4*>(vp + vo) =
          make_uint4(sm.vals_col[c][(4 * g4 + 0) ^ cs], sm.vals_col[c][(4 * g4 + 1) ^ cs],
                     sm.vals_col[c][(4 * g4 + 2) ^ cs], sm.vals_col[c][(4 * g4 + 3) ^ cs]);
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) word |= ((sm.bnibs[4 * g4 + q][c >> 2] >> sh) & 0xFu) << (4 * q);
      mp[mo] = (uint16_t)word;
    }
  }
}

// Coalesced stores of a staged tile: 16-byte row and column segments, each
// contiguous in the forms' blocked order (its columns stay in one block).
__device__ __forceinline__ void write_tile(const TileRef& tr, int tid, const CompressSmem& sm) {
  if (tr.rows == kTile && tr.cols == kTile) {
    write_full_tile(tr, tid, sm);
    return;
  }
  const ScJob& jb = tr.jb;
  const int64_t R = jb.R, C = jb.C, r0 = tr.r0, c0 = tr.c0;
  const int rows = tr.rows, cols = tr.cols, nbc_t = cols / 4, nbr_t = rows / 4;
  if (jb.idx_out) {
    for (int i = tid; i < nbr_t * (nbc_t / 4); i += kCompressThreads) {
      const int bi = i / (nbc_t / 4), b4 = i - bi * (nbc_t / 4);
      const uint32_t v = (uint32_t)sm.idx[bi][4 * b4] | (uint32_t)sm.idx[bi][4 * b4 + 1] << 8 |
                         (uint32_t)sm.idx[bi][4 * b4 + 2] << 16 | (uint32_t)sm.idx[bi][4 * b4 + 3] << 24;
      *reinterpret_cast<uint32_t*>(jb.idx_out + (r0 / 4 + bi) * (C / 4) + c0 / 4 + 4 * b4) = v;
    }
  }
  if (jb.vals_row) {
    const int q4 = nbc_t / 4;
    for (int i = tid; i < rows * q4; i += kCompressThreads) {
      const int r = i / q4, g4 = i - r * q4;
      const uint4 v = make_uint4(sm.vals_row[r][4 * g4 + 0], sm.vals_row[r][4 * g4 + 1], sm.vals_row[r][4 * g4 + 2],
                                 sm.vals_row[r][4 * g4 + 3]);
      *reinterpret_cast<uint4*>(jb.vals_row + form_off(r0 + r, c0 / 2 + 8 * g4, R, C / 2, kValsBlock)) = v;
      // row r's nibble in each of the four blocks (r/4, 4*g4 + q)
      const int sh = 4 * (r & 3);
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) word |= ((sm.bnibs[r >> 2][4 * g4 + q] >> sh) & 0xFu) << (4 * q);
      jb.meta_row[form_off(r0 + r, c0 / 16 + g4, R, C / 16, kMetaBlock)] = (uint16_t)word;
    }
  }
  if (jb.vals_col) {
    const int q4 = nbr_t / 4;
    for (int i = tid; i < cols * q4; i += kCompressThreads) {
      const int c = i / q4, g4 = i - c * q4, cs = col_swz(c);
      const uint4 v = make_uint4(sm.vals_col[c][(4 * g4 + 0) ^ cs], sm.vals_col[c][(4 * g4 + 1) ^ cs],
                                 sm.vals_col[c][(4 * g4 + 2) ^ cs], sm.vals_col[c][(4 * g4 + 3) ^ cs]);
      *reinterpret_cast<uint4*>(jb.vals_col + form_off(c0 + c, r0 / 2 + 8 * g4, C, R / 2, kValsBlock)) = v;
      // column c's nibble in each of the four blocks (4*g4 + q, c/4)
      const int sh = 16 + 4 * (c & 3);
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) word |= ((sm.bnibs[4 * g4 + q][c >> 2] >> sh) & 0xFu) << (4 * q);
      jb.meta_col[form_off(c0 + c, r0 / 16 + g4, C, R / 16, kMetaBlock)] = (uint16_t)word;
    }
  }
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS accesses have
// completed (lgkmcnt(0)) when it arrives.  __syncthreads() would also wait for
// every outstanding global load and store (vmcnt(0)): with several tiles per
// workgroup, tile 0's search would wait for tile 1's loads, and tile 1's
// staging for tile 0's stores to be acknowledged.  Register results of global
// loads are waited for where they are used, as usual.  The memory clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Each workgroup handles kTilesPerWg tiles.  All of their loads are issued
// first; tile 0 is searched as soon as its own loads land, and tile k+1 is
// searched while the global stores of tile k drain.  A job that counts flips
// gets one atomic add per counter and workgroup, after the tile's waves have
// pooled their counts in LDS.

template <bool kSearch>
__global__ __launch_bounds__(kCompressThreads) void search_compress_kernel(ScJobs jobs) {
  __shared__ CompressSmem sm;
  const int tid = threadIdx.x;
  for (int i = tid; i < (int)(sizeof(PatTable) / 4); i += kCompressThreads)
    reinterpret_cast<uint32_t*>(&sm.pat)[i] = reinterpret_cast<const uint32_t*>(&g_pat)[i];

  // Workgroups are dealt round-robin to the 8 XCDs; remap so each XCD walks a
  // contiguous run of tiles (neighbouring output lines then meet in its L2).
  const int64_t ngroups = (jobs.total_tiles + kTilesPerWg - 1) / kTilesPerWg;
  const int64_t per_xcd = (ngroups + 7) / 8;
  const int64_t grp = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (grp >= ngroups) return;
  // The first four workgroups of each CU (ids below 4 x CUs: the dispatcher
  // fills one slot of every CU before the next) would otherwise all load,
  // then all search, then all store in step, leaving HBM idle while the
  // VALUs work and the reverse.  Starting slot k about k x 2 us late
  // (4096 clocks each) interleaves those phases: 27.8 against 29.9 us for
  // both 1.5B weights (kernel trace, median); 1 or 3 us per slot gave 28.0
  // and 28.4 us.
  if ((int64_t)blockIdx.x < 4 * (int64_t)jobs.cus) {
    const int slot = (int)(blockIdx.x / (unsigned)jobs.cus);
    for (int i = 0; i < slot; ++i) __builtin_amdgcn_s_sleep(64);
  }

  TileRef tr[kTilesPerWg];
  TileData td[kTilesPerWg];
  bool have[kTilesPerWg];
#pragma unroll
  for (int k = 0; k < kTilesPerWg; ++k) {
    const int64_t t = grp * kTilesPerWg + k;
    have[k] = t < jobs.total_tiles;
    // a missing last tile loads the first one again (never staged), which
    // keeps the load sequence the same for every workgroup
    tr[k] = tile_ref(jobs, have[k] ? t : grp * kTilesPerWg);
  }
#pragma unroll
  for (int k = 0; k < kTilesPerWg; ++k)
    if (kSearch && tr[k].jb.idx_prev) load_prev(tr[k], tid, td[k]);
#pragma unroll
  for (int k = 0; k < kTilesPerWg; ++k) load_tile(tr[k], tid, td[k]);
#pragma unroll
  for (int k = 0; k < kTilesPerWg; ++k) {
    if (kSearch && have[k] && tr[k].jb.idx_prev && tid / 8 < tr[k].rows / 4 && 4 * (tid % 8) < tr[k].cols / 4)
      *reinterpret_cast<uint32_t*>(&sm.prev[k][tid / 8][4 * (tid % 8)]) = td[k].prev4;
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < kTilesPerWg; ++k) {
    if (!have[k]) continue;
    const uint32_t f = stage_tile<kSearch>(tr[k], k, tid, td[k], sm);
    if (kSearch && tr[k].jb.flips) {
      const uint32_t w = wave_sum(f);
      if (tid % 64 == 0) sm.flips[k][tid / 64] = w;
    }
    lds_barrier();
    write_tile(tr[k], tid, sm);
    lds_barrier();    // the staging buffer is read out before the next tile overwrites it
  }
  if (kSearch && tid == 0) {
    // one atomic per counter: same-address device atomics serialise, and all
    // workgroups reach this point at about the same time
    unsigned long long* ctr[kTilesPerWg];
    unsigned long long sum[kTilesPerWg];
#pragma unroll
    for (int k = 0; k < kTilesPerWg; ++k) {
      ctr[k] = have[k] ? tr[k].jb.flips : nullptr;
      sum[k] = 0;
      if (ctr[k] == nullptr) continue;
#pragma unroll
      for (int w = 0; w < kCompressWaves; ++w) sum[k] += sm.flips[k][w];
#pragma unroll
      for (int j = 0; j < k; ++j)
        if (ctr[j] == ctr[k]) {
          sum[j] += sum[k];
          sum[k] = 0;
          break;
        }
    }
#pragma unroll
    for (int k = 0; k < kTilesPerWg; ++k)
      if (ctr[k] != nullptr && sum[k] != 0) atomicAdd(ctr[k], sum[k]);
  }
}

// ---------------------------------------------------------------------------
// flip count between two index arrays: 16 blocks per thread per step, at most
// 128 workgroups (one same-address atomic each: those serialise)

constexpr int kFlipThreads = 256;

__global__ __launch_bounds__(kFlipThreads) void flip_count_kernel(const uint8_t* __restrict__ a,
                                                                  const uint8_t* __restrict__ b, int64_t n,
                                                                  unsigned long long* __restrict__ flips) {
  __shared__ uint16_t mask[kNumPatterns];
  __shared__ uint32_t part[kFlipThreads / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < kNumPatterns; i += kFlipThreads) mask[i] = (uint16_t)g_pat.entry[i].y;
  __syncthreads();
  auto diff = [&](uint32_t x, uint32_t y) -> uint32_t {
    x = x < (uint32_t)kNumPatterns ? x : 0u;
    y = y < (uint32_t)kNumPatterns ? y : 0u;
    return (uint32_t)__builtin_popcount((uint32_t)(mask[x] ^ mask[y]));
  };
  uint32_t cnt = 0;
  const int64_t nvec = n / 16;
  const int64_t stride = (int64_t)gridDim.x * kFlipThreads;
  for (int64_t i = (int64_t)blockIdx.x * kFlipThreads + tid; i < nvec; i += stride) {
    const uint4 va = reinterpret_cast<const uint4*>(a)[i];
    const uint4 vb = reinterpret_cast<const uint4*>(b)[i];
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += diff((wa[j] >> (8 * e)) & 0xFF, (wb[j] >> (8 * e)) & 0xFF);
  }
  if (blockIdx.x == 0 && tid < (int)(n - 16 * nvec)) cnt += diff(a[16 * nvec + tid], b[16 * nvec + tid]);
  const uint32_t w = wave_sum(cnt);
  if (tid % 64 == 0) part[tid / 64] = w;
  __syncthreads();
  if (tid == 0) {
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < kFlipThreads / 64; ++k) sum += part[k];
    if (sum) atomicAdd(flips, (unsigned long long)sum);
  }
}

}  // namespace

hipError_t launch_mask_search(const uint16_t* W, int64_t R, int64_t C, uint8_t* idx, hipStream_t s) {
  const int64_t nblocks = (R / 4) * (C / 4);
  if (nblocks == 0) return hipSuccess;
  const int64_t want = (nblocks + kSearchThreads - 1) / kSearchThreads;
  const int64_t grid = want < (1 << 20) ? want : (1 << 20);
  hipLaunchKernelGGL(mask_search_kernel, dim3((unsigned)grid), dim3(kSearchThreads), 0, s, W, R, C, idx);
  return hipGetLastError();
}

hipError_t launch_search_compress_jobs(ScJobs jobs, bool search, hipStream_t s) {
  int64_t total = 0;
  for (int k = 0; k < jobs.count; ++k) {
    ScJob& jb = jobs.j[k];
    jb.tiles_c = (jb.C + kTile - 1) / kTile;
    jb.tile_begin = total;
    total += ((jb.R + kTile - 1) / kTile) * jb.tiles_c;
  }
  jobs.total_tiles = total;
  jobs.cus = (int)device_cu_count();
  if (total == 0) return hipSuccess;
  const int64_t groups = (total + kTilesPerWg - 1) / kTilesPerWg;
  const int64_t grid = ((groups + 7) / 8) * 8;
  if (search)
    hipLaunchKernelGGL(search_compress_kernel<true>, dim3((unsigned)grid), dim3(kCompressThreads), 0, s, jobs);
  else
    hipLaunchKernelGGL(search_compress_kernel<false>, dim3((unsigned)grid), dim3(kCompressThreads), 0, s, jobs);
  return hipGetLastError();
}

hipError_t launch_search_compress(const uint16_t* W, int64_t R, int64_t C, const uint8_t* idx_in,
                                  uint8_t* idx_out, uint16_t* vals_row, uint16_t* meta_row,
                                  uint16_t* vals_col, uint16_t* meta_col, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  ScJobs jobs{};
  jobs.count = 1;
  jobs.j[0] = ScJob{W, R, C, idx_in, idx_out, vals_row, meta_row, vals_col, meta_col, nullptr, nullptr, 0, 0};
  return launch_search_compress_jobs(jobs, idx_in == nullptr, s);
}

hipError_t launch_flip_count(const uint8_t* a, const uint8_t* b, int64_t n, unsigned long long* flips,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n / 16 + kFlipThreads - 1) / kFlipThreads;
  const int64_t grid = want < 1 ? 1 : (want < 128 ? want : 128);
  hipLaunchKernelGGL(flip_count_kernel, dim3((unsigned)grid), dim3(kFlipThreads), 0, s, a, b, n, flips);
  return hipGetLastError();
}

}  // namespace sp24
