// MVUE: minimum-variance unbiased 2:4 pruning of a gradient, streaming kernel.
//
// "Accelerating Transformer Pre-training with 2:4 Sparsity" lists an MVUE
// kernel (reproducibility table, "Software Dependencies" row) and gives no
// more.  The library's estimator keeps 2 of every 4 consecutive entries of a
// row.  For a group a_0..a_3 with S = sum |a_i|, the keep probabilities are
// p_i = 2|a_i| / S, the choice that minimises sum a_i^2 (1/p_i - 1) under
// sum p_i = 2.  An entry with p_k > 1 is capped at 1, and the others then get
// |a_j| / (S - |a_k|).  Two entries are drawn by systematic sampling with the
// group's uniform u (caller-supplied): over the cumulative sums C_0..C_2 of p,
// the picks are the intervals holding u and u + 1.  A kept entry is a_i / p_i,
// so the estimate is unbiased.  A group with fewer than two non-zero entries
// is kept as it is.
//
// Every step is fp32, in a fixed order and without contraction, so the picks
// and values are reproducible bit for bit; the order (mvue_group) compares
// cumulative masses instead of dividing, the same decisions in exact
// arithmetic.  Output: the
// library's 2:4 row form (vals fp16 [rows][cols/2], meta [rows][cols/16], one
// nibble i0 | i1 << 2 per group) in the forms' blocked order, which the sparse
// GEMM consumes directly.
//
// Bound by HBM: per entry it reads 2 bytes of the gradient and 1 of u (4 bytes
// per group) and writes 1.125 bytes, against about 50 VALU operations per
// group.  One lane handles 16 entries (one meta word, 8 halves of vals) with
// 16-byte accesses.  In the blocked order a 64-row band's column block of 64
// entries is 4 KB of vals and 512 B of meta, contiguous, so the lanes are laid
// out to keep both the gradient's reads and the forms' writes in long runs
// (mvue_kernel).  The row-major output of the same kernel design ran about 6%
// faster (69-71 against 72-78 us at 16384 x 6400): the price of handing the
// sparse GEMM its operand order.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kMvueThreads = 256;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Pick {
  uint32_t nib;    // i | k << 2
  float vi, vk;
};

// v[j] for j in 0..3 as two levels of selects on j's bits (a compare chain
// would become a switch, lowered to branches)
__device__ __forceinline__ float sel4(const float (&v)[4], int j) {
  const float lo = (j & 1) ? v[1] : v[0];
  const float hi = (j & 1) ? v[3] : v[2];
  return (j & 2) ? hi : lo;
}

// The probabilities are carried as masses w_j over a scale D (p_j = w_j / D,
// sum w_j = 2D): uncapped, w_j = |a_j| and D = S/2; with entry c capped,
// w_j = |a_j| for j != c and w_c = D = S - |a_c|.  C_j <= u then reads
// W_j <= u D on the cumulative masses W_j, and a kept value a_j / p_j is a_c
// for the capped entry and sign(a_j) D for any other non-zero entry.  No step
// divides, and every choice is a select, so a wave never splits.
__device__ __forceinline__ Pick mvue_group(const float (&a)[4], float u) {
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = __builtin_fabsf(a[j]);
  const float S = ((m[0] + m[1]) + m[2]) + m[3];
  // p_c > 1 <=> 2|a_c| > S.  At most one entry can satisfy it: the rounded
  // running sum S is at least the rounded sum of any two entries, which is
  // at least twice the smaller one.
  bool cap[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cap[j] = 2.0f * m[j] > S;
  const bool capped = (cap[0] | cap[1]) | (cap[2] | cap[3]);
  // the ordered sum of the other three: a zero in the capped slot adds nothing
  float o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = cap[j] ? 0.0f : m[j];
  const float rest = ((o[0] + o[1]) + o[2]) + o[3];
  const float D = capped ? rest : S * 0.5f;
  float w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = cap[j] ? D : m[j];
  const float W0 = w[0], W1 = W0 + w[1], W2 = W1 + w[2];
  const float uD = u * D, uD1 = uD + D;
  int i = (int)(W0 <= uD) + (int)(W1 <= uD) + (int)(W2 <= uD);
  int k = (int)(W0 <= uD1) + (int)(W1 <= uD1) + (int)(W2 <= uD1);
  // rounding can put u and u + 1 in one interval: take the next one, or
  // (2, 3) from the last
  const bool same = k == i;
  k = same ? (i < 3 ? i + 1 : 3) : k;
  i = same && i == 3 ? 2 : i;
  // fewer than two non-zero entries: keep the non-zero one (if any) and the
  // lowest other index, both exactly
  const int nz = (int)(m[0] != 0.0f) + (int)(m[1] != 0.0f) + (int)(m[2] != 0.0f) + (int)(m[3] != 0.0f);
  const bool few = nz < 2;
  const int only = m[1] != 0.0f ? 1 : m[2] != 0.0f ? 2 : m[3] != 0.0f ? 3 : 1;
  i = few ? 0 : i;
  k = few ? (m[0] != 0.0f ? 1 : only) : k;
  const uint32_t capbits = (uint32_t)cap[0] | (uint32_t)cap[1] << 1 | (uint32_t)cap[2] << 2 | (uint32_t)cap[3] << 3;
  // the kept values, computed for the two picks only
  // (sign(a_j) D, or +0 for a zero a_j, built from the bits)
  const uint32_t dbits = __builtin_bit_cast(uint32_t, D);
  auto value = [&](int j) {
    const uint32_t ab = __builtin_bit_cast(uint32_t, sel4(a, j));
    const bool exact = few | (((capbits >> j) & 1u) != 0);
    const uint32_t nonzero = 0u - (uint32_t)((ab << 1) != 0u);
    const uint32_t est = (dbits | (ab & 0x80000000u)) & nonzero;
    return __builtin_bit_cast(float, exact ? ab : est);
  };
  Pick r;
  r.nib = (uint32_t)(i | (k << 2));
  r.vi = value(i);
  r.vk = value(k);
  return r;
}

// Workgroup b: band b / regions (rows 64 k ..) and words 16 (b % regions) ..
// + 15 of each of its rows, i.e. four column blocks, whose outputs are one
// 16 KB run of vals.  Lane l of wave v takes word l % 16 of rows
// 4 v + l / 16 + 16 i: each wave instruction reads 512 contiguous bytes of
// the gradient from each of 4 rows and writes 256 contiguous bytes (4 rows)
// into each of the 4 blocks.  (One block per workgroup, 16 rows x 128 B per
// wave instruction, ran 10-15% slower; 2 rows x 1 KB, which writes 128-byte
// runs, and one row of 2 KB, which writes 64-byte runs, slower still.)
constexpr int kMvueWords = 16;   // words of a row per region
__global__ __launch_bounds__(kMvueThreads) void mvue_kernel(const uint16_t* __restrict__ M, const float* __restrict__ U,
                                                            int64_t rows, int64_t cols, uint32_t regions,
                                                            uint16_t* __restrict__ vals,
                                                            uint16_t* __restrict__ meta) {
  constexpr int kRowsPerWave = 64 / kMvueWords, kRowsPerPass = kRowsPerWave * (kMvueThreads / 64);
  const uint32_t b = blockIdx.x, band = b / regions, reg = b - band * regions;
  const int64_t m = cols / 16;   // meta words (16-entry segments) per row
  const int64_t r0 = 64 * (int64_t)band;
  const int h = (int)min<int64_t>(64, rows - r0);
  const int lane = (int)(threadIdx.x & 63), wave = (int)(threadIdx.x >> 6);
  const int64_t seg = (int64_t)kMvueWords * reg + lane % kMvueWords;
  if (seg >= m) return;
  // the segment's column block j (4 words, w of them in a row's last block)
  // and the blocked-order index of its row 0 in the band
  const int64_t j = seg >> 2;
  const int w = (int)min<int64_t>(4, m - 4 * j);
  const int64_t blk = r0 * m + 4 * j * h + (seg & 3);
#pragma unroll 2
  for (int rr = wave * kRowsPerWave + lane / kMvueWords; rr < h; rr += kRowsPerPass) {
    const int64_t r = r0 + rr;
    const int64_t out = blk + (int64_t)rr * w;
    const u32x4* src = reinterpret_cast<const u32x4*>(M + r * cols + 16 * seg);
    const h8 lo = __builtin_bit_cast(h8, __builtin_nontemporal_load(src));
    const h8 hi = __builtin_bit_cast(h8, __builtin_nontemporal_load(src + 1));
    const f32x4 us = *reinterpret_cast<const f32x4*>(U + r * (cols / 4) + 4 * seg);
    h8 o;
    uint32_t word = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = (float)(g < 2 ? lo[4 * g + e] : hi[4 * (g - 2) + e]);
      const Pick pk = mvue_group(a, us[g]);
      o[2 * g] = (_Float16)pk.vi;
      o[2 * g + 1] = (_Float16)pk.vk;
      word |= pk.nib << (4 * g);
    }
    *(reinterpret_cast<u32x4*>(vals) + out) = __builtin_bit_cast(u32x4, o);
    meta[out] = (uint16_t)word;
  }
}

}  // namespace

hipError_t launch_mvue(const uint16_t* M, const float* U, int64_t rows, int64_t cols, uint16_t* vals, uint16_t* meta,
                       hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t regions = (cols / 16 + kMvueWords - 1) / kMvueWords, bands = (rows + 63) / 64;
  hipLaunchKernelGGL(mvue_kernel, dim3((unsigned)(bands * regions)), dim3(kMvueThreads), 0, s, M, U, rows, cols,
                     (uint32_t)regions, vals, meta);
  return hipGetLastError();
}

}  // namespace sp24
