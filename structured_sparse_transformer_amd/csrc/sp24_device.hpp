// Device helpers shared by the GEMM kernels: raw buffer descriptors and
// direct global->LDS loads for gfx950, and the device's CU count.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace sp24 {

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, gfx9 family

// Raw buffer descriptor over [base, base + bytes), kept in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = (int)kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// Direct global->LDS loads: lane l's bytes land at LDS address M0 + l * size.
// Written as asm so that the compiler's wait-count pass does not make every
// later LDS read wait for all outstanding loads (it cannot tell the stage
// buffers apart); completion is tracked with explicit vmcnt waits instead.
// The LDS address is an input bound to M0, so the compiler sets M0; the asm
// has no register outputs, and its s_nop 0 covers the M0-write hazard.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t lds, int voffset) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voffset), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma_b32(i32x4 rsrc, uint32_t lds, int voffset) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" : : "v"(voffset), "s"(rsrc), "{m0}"(lds) : "memory");
}

// GELU(x) = x * Phi(x), Phi(x) = erfc(-x / sqrt 2) / 2: the erfc form keeps
// its relative accuracy for negative x, where 1 + erf(x / sqrt 2) cancels to
// zero in fp32 (below about x = -5.3).  Shared by the GEGLU kernels and the
// fused GEGLU epilogue of the forward GEMM.
//
// erfc(z), z = |x| / sqrt 2 >= 0, is evaluated as t * exp(-z^2 + P(t)) with
// t = 1 / (1 + z/2), the form of the Chebyshev erfc in Numerical Recipes
// (section 6.2).  P is a degree-9 polynomial fitted here (weighted least
// squares, gen_erfc_fit.py) to log(erfcx(z) / t) over t in [0, 1]; its largest
// error, with the coefficients rounded to fp32, is 1.2e-7.
//
// The exponent reaches -z^2 = -x^2/2 (about -18 at x = -6), where its fp32
// rounding alone would cost about 1e-6 relative.  So it is carried as s + e:
// x^2 is split exactly by an FMA, and s = -x^2/2 + P comes with its rounding
// error (Fast2Sum, exact once |x^2/2| >= |P|, which is where it matters).
// exp(s + e) = 2^(s log2 e) * (1 + e'), where the hardware 2^y takes the
// rounded product and e' gathers e and the product's error.  Emulated in fp32
// over every fp16 x, with 2^y off by up to 2 ulp, Phi is within 7e-7
// relative (tests/test_gelu_host_model.py).
constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kErfcP[10] = {-1.2655122f, 1.0000226f, 0.37412503f,  0.096388236f, -0.18396664f,
                              0.27135256f, -1.1211007f, 1.473255f, -0.8133247f,  0.1687606f};
constexpr float kLog2E = 1.442695f, kLog2ELo = 1.925963e-08f, kLn2 = 0.6931472f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
// erfc / 2 = t exp(-z^2 + P(t) - ln 2): the halving rides in the constant
// term (its fp32 rounding adds at most 6e-8 to the exponent).
constexpr float kErfcP0Half = kErfcP[0] - kLn2;
struct ErfcParts {
  float half;   // erfc(|x| / sqrt 2) / 2
  float p;      // P(t) - ln 2
  float ex;     // exp(-x^2/2 + P(t) - ln 2)
};
// The argument is clamped to [-64, 64]: beyond it erfc(|x| / sqrt 2) / 2 is
// 0 in fp32 either way, and x = +-inf would otherwise turn x^2's split into
// inf - inf.  GELU's final multiply by the unclamped x keeps +inf -> +inf and
// -inf -> NaN (x Phi(x) = -inf * 0), as in exact arithmetic in IEEE.
__device__ __forceinline__ ErfcParts erfc_parts(float xin) {
  const float x = __builtin_amdgcn_fmed3f(xin, -64.0f, 64.0f);
  const float z = __builtin_fabsf(x) * kInvSqrt2;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
  float p = kErfcP[9];
#pragma unroll
  for (int k = 8; k >= 1; --k) p = __builtin_fmaf(p, t, kErfcP[k]);
  p = __builtin_fmaf(p, t, kErfcP0Half);
  const float hi = x * x;
  const float lo = __builtin_fmaf(x, x, -hi);
  const float a = -0.5f * hi;
  const float s = a + p;
  const float e = __builtin_fmaf(-0.5f, lo, p - (s - a));
  const float yh = s * kLog2E;
  const float yl = __builtin_fmaf(s, kLog2ELo, __builtin_fmaf(s, kLog2E, -yh));
  const float E = __builtin_amdgcn_exp2f(yh);
  ErfcParts r;
  r.ex = __builtin_fmaf(E, __builtin_fmaf(yl, kLn2, e), E);
  r.half = t * r.ex;
  r.p = p;
  return r;
}
__device__ __forceinline__ float gelu_cdf(float x) {
  const ErfcParts r = erfc_parts(x);
  return x < 0.0f ? r.half : 1.0f - r.half;
}
// Phi(x) and phi(x) = exp(-x^2/2) / sqrt(2 pi) together.  phi reuses the
// exponential above, exp(-x^2/2) = ex * exp(-p); p lies in [-1.96, -0.69],
// so exp(-p) needs no extra care (within 7.5e-7 relative in the same
// emulation).
__device__ __forceinline__ void gelu_cdf_pdf(float x, float& cdf, float& pdf) {
  const ErfcParts r = erfc_parts(x);
  cdf = x < 0.0f ? r.half : 1.0f - r.half;
  pdf = (r.ex * __builtin_amdgcn_exp2f(-r.p * kLog2E)) * kInvSqrt2Pi;
}
__device__ __forceinline__ float gelu_f32(float x) { return x * gelu_cdf(x); }
// value * GELU(gate) from fp16 inputs: the fp32 product, rounded to nearest
// even in fp16.  The empty asm pins the product as an fp32 value.  Without
// it the backend may fold the multiply and the conversion into one mixed
// fp16 FMA (v_fma_mixlo_f16), which rounds once instead of twice; it did so
// in the fused GEMM epilogue but not in the GEGLU kernel, and near fp16
// rounding ties the two then differed by one ulp.
__device__ __forceinline__ _Float16 geglu_f16(_Float16 value, _Float16 gate) {
  float prod = (float)value * gelu_f32((float)gate);
  asm volatile("" : "+v"(prod));
  return (_Float16)prod;
}

// Number of compute units of the current device (cached per device; host
// threads may race to fill an entry, and all of them store the same value).
inline int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace sp24
