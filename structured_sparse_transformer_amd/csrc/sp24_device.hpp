// Device helpers shared by the GEMM kernels: raw buffer descriptors and
// direct global->LDS loads for gfx950, and the device's CU count.
#pragma once
#include <hip/hip_runtime.h>
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
// fused GEGLU epilogue of the forward GEMM, so that both give identical bits.
constexpr float kInvSqrt2 = 0.70710678118654752440f;
__device__ __forceinline__ float gelu_cdf(float x) { return 0.5f * erfcf(-x * kInvSqrt2); }
__device__ __forceinline__ float gelu_f32(float x) { return x * gelu_cdf(x); }
// value * GELU(gate) from fp16 inputs, rounded to nearest even in fp16
__device__ __forceinline__ _Float16 geglu_f16(_Float16 value, _Float16 gate) {
  return (_Float16)((float)value * gelu_f32((float)gate));
}

// Number of compute units of the current device (cached per device).
inline int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace sp24
