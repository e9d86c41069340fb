// Transposable 2:4 pattern tables, built at compile time.
//
// A transposable 2:4 mask keeps two of four entries in every row and every
// column of a 4x4 block ("Accelerating Transformer Pre-training with 2:4
// Sparsity", abstract; Algorithm 1 takes the set of such patterns as its
// input m).  Patterns are numbered by the tuple (a, b, c, d) of row-pair codes
// of rows 0..3 in lexicographic order, with codes 0:{0,1} 1:{0,2} 2:{0,3}
// 3:{1,2} 4:{1,3} 5:{2,3}; there are 90 of them.
//
// Besides the plain masks, the tables here drive the fast exact search
// (search_fast in sp24_search.hip).  A pattern's score splits into a "top"
// part (rows 0, 1: codes a, b) and a "bottom" part (rows 2, 3: codes c, d).
// The top pair leaves a column deficit r = 2 - colcount(a, b), and the bottom
// pair must fill it exactly: colcount(c, d) = r.  There are 19 such deficit
// classes.  For each top pair, `top_base` is the index of the first pattern
// with that prefix; for each bottom pair, `bot_rank` is its rank among the
// bottom pairs of its class in lexicographic order.  The index of pattern
// (a, b, c, d) is then top_base(a, b) + bot_rank(c, d).
#pragma once
#include <cstdint>

namespace sp24 {

constexpr int kNumPatterns = 90;
constexpr int kNumClasses = 19;

// column pair kept by row-pair code k
constexpr int kPairLo[6] = {0, 0, 0, 1, 1, 2};
constexpr int kPairHi[6] = {1, 2, 3, 2, 3, 3};

struct PatternTables {
  uint16_t mask[kNumPatterns];       // bit 4r+c set when (r, c) is kept
  uint16_t row_nib[kNumPatterns];    // nibble of row r at bits 4r: i0 | i1 << 2
  uint16_t col_nib[kNumPatterns];    // nibble of column c at bits 4c
  uint8_t code[kNumPatterns][4];     // row-pair codes (a, b, c, d)
  // pair (x, y) of row-pair codes, x slowest: 36 entries
  int8_t pair_class[36];             // deficit class of a top pair (rows 0,1)
  int8_t bot_class[36];              // class of a bottom pair (rows 2,3); same ids
  uint8_t top_base[36];              // first pattern index with prefix (a, b)
  uint8_t bot_rank[36];              // rank of (c, d) within its class
  uint8_t class_size[kNumClasses];
};

constexpr int colcount_pair(int x, int y, int col) {
  return (kPairLo[x] == col || kPairHi[x] == col ? 1 : 0) +
         (kPairLo[y] == col || kPairHi[y] == col ? 1 : 0);
}

// Deficit vector r in {0,1,2}^4 with sum 4, encoded base 3.
constexpr int deficit_code(int x, int y) {
  int v = 0;
  for (int col = 3; col >= 0; --col) v = v * 3 + (2 - colcount_pair(x, y, col));
  return v;
}
constexpr int fill_code(int x, int y) {
  int v = 0;
  for (int col = 3; col >= 0; --col) v = v * 3 + colcount_pair(x, y, col);
  return v;
}

constexpr PatternTables build_tables() {
  PatternTables t{};
  int n = 0;
  for (int a = 0; a < 6; ++a)
    for (int b = 0; b < 6; ++b)
      for (int c = 0; c < 6; ++c)
        for (int d = 0; d < 6; ++d) {
          const int codes[4] = {a, b, c, d};
          int cnt[4] = {0, 0, 0, 0};
          for (int r = 0; r < 4; ++r) {
            cnt[kPairLo[codes[r]]]++;
            cnt[kPairHi[codes[r]]]++;
          }
          if (cnt[0] != 2 || cnt[1] != 2 || cnt[2] != 2 || cnt[3] != 2) continue;
          uint16_t m = 0, rn = 0;
          for (int r = 0; r < 4; ++r) {
            const int lo = kPairLo[codes[r]], hi = kPairHi[codes[r]];
            m |= (uint16_t)((1u << (4 * r + lo)) | (1u << (4 * r + hi)));
            rn |= (uint16_t)((lo | (hi << 2)) << (4 * r));
            t.code[n][r] = (uint8_t)codes[r];
          }
          uint16_t cn = 0;
          for (int col = 0; col < 4; ++col) {
            int first = -1, second = -1;
            for (int r = 0; r < 4; ++r)
              if (m & (1u << (4 * r + col))) {
                if (first < 0) first = r; else second = r;
              }
            cn |= (uint16_t)((first | (second << 2)) << (4 * col));
          }
          t.mask[n] = m;
          t.row_nib[n] = rn;
          t.col_nib[n] = cn;
          ++n;
        }
  // deficit classes, numbered in order of first appearance among top pairs
  int class_of_code[81];
  for (int i = 0; i < 81; ++i) class_of_code[i] = -1;
  int ncls = 0;
  for (int x = 0; x < 6; ++x)
    for (int y = 0; y < 6; ++y) {
      const int dc = deficit_code(x, y);
      if (class_of_code[dc] < 0) class_of_code[dc] = ncls++;
      t.pair_class[6 * x + y] = (int8_t)class_of_code[dc];
    }
  for (int x = 0; x < 6; ++x)
    for (int y = 0; y < 6; ++y) t.bot_class[6 * x + y] = (int8_t)class_of_code[fill_code(x, y)];
  for (int k = 0; k < kNumClasses; ++k) t.class_size[k] = 0;
  for (int p = 0; p < 36; ++p) {
    // bottom pairs are visited in lexicographic order, so the running count
    // of a class is the rank of the pair within it
    t.bot_rank[p] = t.class_size[t.bot_class[p]]++;
  }
  for (int p = 0; p < 36; ++p) t.top_base[p] = 0xFF;
  for (int i = n - 1; i >= 0; --i) t.top_base[6 * t.code[i][0] + t.code[i][1]] = (uint8_t)i;
  return t;
}

constexpr PatternTables kTables = build_tables();

constexpr bool tables_ok() {
  int n = 0;
  for (int i = 0; i < kNumPatterns; ++i) n += kTables.mask[i] != 0;
  bool ok = n == kNumPatterns;
  for (int p = 0; p < 36; ++p) ok = ok && kTables.top_base[p] < kNumPatterns && kTables.pair_class[p] >= 0 &&
                                    kTables.bot_class[p] >= 0 && kTables.bot_class[p] < kNumClasses;
  // every class has as many top pairs as bottom pairs (the two halves mirror)
  for (int k = 0; k < kNumClasses; ++k) {
    int tops = 0;
    for (int p = 0; p < 36; ++p) tops += kTables.pair_class[p] == k;
    ok = ok && tops == kTables.class_size[k];
  }
  // index decomposition: pattern (a,b,c,d) = top_base(a,b) + bot_rank(c,d)
  for (int i = 0; i < kNumPatterns; ++i) {
    const int tp = 6 * kTables.code[i][0] + kTables.code[i][1];
    const int bp = 6 * kTables.code[i][2] + kTables.code[i][3];
    ok = ok && kTables.top_base[tp] + kTables.bot_rank[bp] == i &&
         kTables.pair_class[tp] == kTables.bot_class[bp];
  }
  return ok;
}
static_assert(tables_ok(), "pattern tables are inconsistent");
static_assert(kTables.mask[0] == 0xCC33 && kTables.mask[89] == 0x33CC, "pattern order");

}  // namespace sp24
