// GEGLU forward and backward, streaming kernels.
//
// "Accelerating Transformer Pre-training with 2:4 Sparsity" names the
// acceleration of gated activation functions (abstract) and a GEGLU kernel
// (reproducibility table, "Software Dependencies" row) without further
// detail.  The library's operation: out = value * GELU(gate), GELU the exact
// x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), on the first linear's output
// U [T, 2h], whose columns come in blocks of G value columns followed by the G
// matching gate columns.  With a small G (16, say) a value and its gate share
// a 128-byte line, so the pair is fetched together; G = h is the plain
// two-halves layout, where they sit h columns apart.
//
// Per hidden unit and token the forward moves 6 bytes (read value and gate,
// write out) and the backward 10 (read value, gate and dOut, write both
// gradients).  At these rates the kernels sit between the HBM roof and the
// fp32 vector roof.  Each lane
// handles 8 consecutive hidden units of one token with 16-byte loads and
// stores; arithmetic is fp32, with results rounded to nearest even in fp16.
// The token and block of a lane come from multiply-shift divisions by
// divisors fixed on the host (make_div).
// Phi and phi come from gelu_cdf / gelu_cdf_pdf (sp24_device.hpp): a fitted
// erfc with one reciprocal and one exponential, about 35 VALU operations.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "sp24_device.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kActThreads = 256;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// streaming 16-byte accesses: every byte is touched once
__device__ __forceinline__ h8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(h8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void st16(uint16_t* p, h8 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

// Division by a divisor d fixed for the launch (1 <= d < 2^31), for
// dividends n < 2^31: floor(n / d) = floor(n * m / 2^(31 + s)) with
// s = ceil(log2 d) and m = ceil(2^(31 + s) / d) < 2^32 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994,
// Theorem 4.2: m d - 2^(31+s) < d <= 2^s).  One 32x32 -> 64-bit multiply and
// a shift, where a division by a kernel argument costs a float reciprocal
// sequence of a dozen VALU operations.
struct DivU31 {
  uint32_t m;
  uint32_t shift;   // 31 + s
};
DivU31 make_div(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  return {(uint32_t)((((uint64_t)1 << (31 + s)) + d - 1) / d), 31 + s};
}
__device__ __forceinline__ uint32_t div_u31(uint32_t n, DivU31 d) {
  return (uint32_t)(((uint64_t)n * d.m) >> d.shift);
}

// One lane per vector of 8 hidden units of one token: vector i is token
// i / (h/8), units 8*(i % (h/8)) ..  Offsets into U and out:
struct Pos {
  int64_t u_val, u_gate, o;
};
// Index is uint32_t (with the multiply-shift divisions) when the vector count
// is below 2^31, else uint64_t with plain divisions.
struct Geom32 {
  uint32_t hv, group;
  DivU31 by_hv, by_group;
};
struct Geom64 {
  uint64_t hv, group;
};
__device__ __forceinline__ Pos position(uint32_t i, const Geom32& g) {
  const uint32_t t = div_u31(i, g.by_hv), unit = (i - t * g.hv) * 8;
  const uint32_t b = div_u31(unit, g.by_group), w = unit - b * g.group;
  Pos p;
  p.u_val = (int64_t)t * 2 * (int64_t)g.hv * 8 + (int64_t)(2 * g.group * b + w);
  p.u_gate = p.u_val + (int64_t)g.group;
  p.o = (int64_t)t * (int64_t)g.hv * 8 + (int64_t)unit;
  return p;
}
__device__ __forceinline__ Pos position(uint64_t i, const Geom64& g) {
  const uint64_t t = i / g.hv, unit = (i - t * g.hv) * 8;
  const uint64_t b = unit / g.group, w = unit - b * g.group;
  Pos p;
  p.u_val = (int64_t)t * 2 * (int64_t)g.hv * 8 + (int64_t)(2 * g.group * b + w);
  p.u_gate = p.u_val + (int64_t)g.group;
  p.o = (int64_t)t * (int64_t)g.hv * 8 + (int64_t)unit;
  return p;
}

template <typename Index, typename Geom>
__global__ __launch_bounds__(kActThreads) void geglu_fwd_kernel(const uint16_t* __restrict__ U, Index n, Geom geom,
                                                               uint16_t* __restrict__ out) {
  const Index i = (Index)blockIdx.x * kActThreads + threadIdx.x;
  if (i >= n) return;
  const Pos p = position(i, geom);
  const h8 v = ld16(U + p.u_val);
  const h8 g = ld16(U + p.u_gate);
  h8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = geglu_f16(v[e], g[e]);
  st16(out + p.o, o);
}

// The backward's two output vectors of a lane sit `group` columns apart, so
// with groups below 64 columns each store instruction covers only part of
// every 128-byte line it touches.  Streamed out as such (non-temporal) those
// partial lines cost a quarter of the kernel's time.  When the group divides
// 512, a full wave's 64 vectors are 512 consecutive hidden units whose value
// and gate gradients fill one exclusive 2 KB span of dU, so the wave stages
// them in LDS and writes the span as two contiguous 1 KB stores.  Otherwise
// (and for a last, partial wave) each lane stores its own vectors, as
// ordinary stores that L2 merges into whole lines.
template <typename Index, typename Geom>
__global__ __launch_bounds__(kActThreads) void geglu_bwd_kernel(const uint16_t* __restrict__ U,
                                                               const uint16_t* __restrict__ dout, Index n, Geom geom,
                                                               uint16_t* __restrict__ dU, bool staged) {
  __shared__ __align__(16) unsigned char stage[kActThreads / 64][2048];
  const Index i = (Index)blockIdx.x * kActThreads + threadIdx.x;
  const Index w0 = i - (Index)(threadIdx.x & 63);   // the wave's first vector
  const bool whole = staged && w0 + 64 <= n;          // uniform across the wave
  if (i >= n) return;
  const Pos p = position(i, geom);
  const h8 v = ld16(U + p.u_val);
  const h8 g = ld16(U + p.u_gate);
  const h8 d = ld16(dout + p.o);
  h8 dv, dg;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (float)g[e], dy = (float)d[e];
    float cdf, pdf;
    gelu_cdf_pdf(x, cdf, pdf);
    dv[e] = (_Float16)(dy * (x * cdf));
    dg[e] = (_Float16)(dy * (float)v[e] * (cdf + x * pdf));
  }
  if (whole) {
    // vector j covers flattened hidden units 8j .. 8j+7, and a block of
    // `group` such units occupies 2 * group columns of dU, so the wave's
    // units [8 w0, 8 w0 + 512) are dU's [16 w0, 16 w0 + 1024)
    unsigned char* st = stage[threadIdx.x >> 6];
    const int64_t base = (int64_t)w0 * 16;
    *reinterpret_cast<h8*>(st + (p.u_val - base) * 2) = dv;
    *reinterpret_cast<h8*>(st + (p.u_gate - base) * 2) = dg;
    __builtin_amdgcn_wave_barrier();
    const int lane = threadIdx.x & 63;
    const u32x4 a = *reinterpret_cast<const u32x4*>(st + lane * 16);
    const u32x4 b = *reinterpret_cast<const u32x4*>(st + 1024 + lane * 16);
    st16(dU + base + lane * 8, __builtin_bit_cast(h8, a));
    st16(dU + base + 512 + lane * 8, __builtin_bit_cast(h8, b));
  } else {
    *reinterpret_cast<u32x4*>(dU + p.u_val) = __builtin_bit_cast(u32x4, dv);
    *reinterpret_cast<u32x4*>(dU + p.u_gate) = __builtin_bit_cast(u32x4, dg);
  }
}

}  // namespace

namespace {
// 32-bit geometry when every index fits below 2^31: the vector index (lanes
// past n included, up to the grid's end) and the unit offset below h.
bool fits31(int64_t n, int64_t h) { return n + kActThreads < ((int64_t)1 << 31) && h < ((int64_t)1 << 31); }
Geom32 geom32(int64_t h, int64_t group) {
  return {(uint32_t)(h / 8), (uint32_t)group, make_div((uint32_t)(h / 8)), make_div((uint32_t)group)};
}
}  // namespace

hipError_t launch_geglu_fwd(const uint16_t* U, int64_t T, int64_t h, int64_t group, uint16_t* out, hipStream_t s) {
  const int64_t n = T * (h / 8);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kActThreads - 1) / kActThreads));
  if (fits31(n, h))
    hipLaunchKernelGGL((geglu_fwd_kernel<uint32_t, Geom32>), grid, dim3(kActThreads), 0, s, U, (uint32_t)n,
                       geom32(h, group), out);
  else
    hipLaunchKernelGGL((geglu_fwd_kernel<uint64_t, Geom64>), grid, dim3(kActThreads), 0, s, U, (uint64_t)n,
                       Geom64{(uint64_t)(h / 8), (uint64_t)group}, out);
  return hipGetLastError();
}

hipError_t launch_geglu_bwd(const uint16_t* U, const uint16_t* dout, int64_t T, int64_t h, int64_t group,
                            uint16_t* dU, hipStream_t s) {
  const int64_t n = T * (h / 8);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kActThreads - 1) / kActThreads));
  // groups of 64 columns or more already fill whole lines per instruction
  const bool staged = group < 64 && 512 % group == 0;
  if (fits31(n, h))
    hipLaunchKernelGGL((geglu_bwd_kernel<uint32_t, Geom32>), grid, dim3(kActThreads), 0, s, U, dout, (uint32_t)n,
                       geom32(h, group), dU, staged);
  else
    hipLaunchKernelGGL((geglu_bwd_kernel<uint64_t, Geom64>), grid, dim3(kActThreads), 0, s, U, dout, (uint64_t)n,
                       Geom64{(uint64_t)(h / 8), (uint64_t)group}, dU, staged);
  return hipGetLastError();
}

}  // namespace sp24
