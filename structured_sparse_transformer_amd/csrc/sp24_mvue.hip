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
// Every step is fp32, in a fixed order, with IEEE division and no contraction,
// so the picks and values are reproducible bit for bit.  Output: the
// library's 2:4 row form (vals fp16 [rows][cols/2], meta [rows][cols/16], one
// nibble i0 | i1 << 2 per group), which the sparse GEMM consumes directly.
//
// Bound by HBM: per entry it reads 2 bytes of the gradient and 1 of u (4 bytes
// per group) and writes 1.125 bytes.  One lane handles 16 entries (one meta
// word) with 16-byte accesses.
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

__device__ __forceinline__ Pick mvue_group(const float (&a)[4], float u) {
  float m[4];
  int nz = 0, first_nz = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = __builtin_fabsf(a[i]);
    if (m[i] != 0.0f) {
      if (first_nz < 0) first_nz = i;
      ++nz;
    }
  }
  Pick r;
  if (nz < 2) {
    int i = first_nz < 0 ? 0 : first_nz;
    int k = i == 0 ? 1 : 0;
    if (k < i) {
      const int t = i;
      i = k;
      k = t;
    }
    r.nib = (uint32_t)(i | (k << 2));
    r.vi = a[i];
    r.vk = a[k];
    return r;
  }
  const float S = ((m[0] + m[1]) + m[2]) + m[3];
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (2.0f * m[i]) / S;
  int kc = -1;
#pragma unroll
  for (int i = 3; i >= 0; --i)
    if (p[i] > 1.0f) kc = i;
  if (kc >= 0) {
    float rest = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j != kc) rest = rest + m[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = j == kc ? 1.0f : m[j] / rest;
  }
  const float C0 = p[0], C1 = C0 + p[1], C2 = C1 + p[2];
  const float u1 = u + 1.0f;
  int i = (C0 <= u) + (C1 <= u) + (C2 <= u);
  int k = (C0 <= u1) + (C1 <= u1) + (C2 <= u1);
  if (k == i) {
    if (i < 3) {
      k = i + 1;
    } else {
      i = 2;
      k = 3;
    }
  }
  r.nib = (uint32_t)(i | (k << 2));
  r.vi = p[i] > 0.0f ? a[i] / p[i] : 0.0f;
  r.vk = p[k] > 0.0f ? a[k] / p[k] : 0.0f;
  return r;
}

template <typename Index>
__global__ __launch_bounds__(kMvueThreads) void mvue_kernel(const uint16_t* __restrict__ M, const float* __restrict__ U,
                                                            Index n, uint16_t* __restrict__ vals,
                                                            uint16_t* __restrict__ meta) {
  // lane i: entries 16i .. 16i+15 of the flattened matrix (rows are whole
  // multiples of 16 entries, so a lane never straddles two rows)
  const Index i = (Index)blockIdx.x * kMvueThreads + threadIdx.x;
  if (i >= n) return;
  const h8 lo = __builtin_bit_cast(h8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(M) + 2 * (int64_t)i));
  const h8 hi =
      __builtin_bit_cast(h8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(M) + 2 * (int64_t)i + 1));
  const f32x4 us = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(U) + (int64_t)i);
  h8 out;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (float)(g < 2 ? lo[4 * g + e] : hi[4 * (g - 2) + e]);
    const Pick pk = mvue_group(a, us[g]);
    out[2 * g] = (_Float16)pk.vi;
    out[2 * g + 1] = (_Float16)pk.vk;
    word |= pk.nib << (4 * g);
  }
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, out), reinterpret_cast<u32x4*>(vals) + (int64_t)i);
  meta[i] = (uint16_t)word;
}

}  // namespace

hipError_t launch_mvue(const uint16_t* M, const float* U, int64_t rows, int64_t cols, uint16_t* vals, uint16_t* meta,
                       hipStream_t s) {
  const int64_t n = rows * (cols / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kMvueThreads - 1) / kMvueThreads));
  if (n < ((int64_t)1 << 32) - kMvueThreads)
    hipLaunchKernelGGL(mvue_kernel<uint32_t>, grid, dim3(kMvueThreads), 0, s, M, U, (uint32_t)n, vals, meta);
  else
    hipLaunchKernelGGL(mvue_kernel<uint64_t>, grid, dim3(kMvueThreads), 0, s, M, U, (uint64_t)n, vals, meta);
  return hipGetLastError();
}

}  // namespace sp24
