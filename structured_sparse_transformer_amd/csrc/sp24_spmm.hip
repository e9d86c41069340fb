// 2:4 sparse x dense GEMM for gfx950 sparse matrix cores (SMFMAC).
//
// Computes out[T][N] = A[T][K] * S[N][K]^T where S is 2:4 sparse along K and
// stored in the library's row form (vals [N][K/2] fp16, meta [N][K/16] with
// one nibble i0 | i1 << 2 per group of 4).  One kernel serves both FFN GEMMs
// of "Accelerating Transformer Pre-training with 2:4 Sparsity" (abstract: 2:4
// sparse matrix multiplication for the feed-forward layers; reproducibility
// table, "Software Dependencies" row: the 2:4 sparse MMs):
//   forward         Y  = X  Ws^T : A = X,  S = row form of W    (N = R, K = C)
//   input gradient  dX = dY Ws   : A = dY, S = column form of W (N = C, K = R)
// The column form exists because the mask is transposable, so the input
// gradient runs on the sparse matrix cores too.
//
// Sparse MFMA v_smfmac_f32_32x32x32_f16 computes D[32x32] += S[32x32] * B[32x32]
// with S compressed to 32x16.  Operand layout (lane l, g = l / 32):
//   S: row l % 32, dense k in [16g, 16g + 16): 8 kept fp16 values in order and
//      their 16-bit index word, which is exactly one meta word of the row form;
//   B: column l % 32, k in [8g, 8g + 8) then [16 + 8g, 16 + 8g + 8);
//   D: column l % 32, rows 8*(i/4) + 4g + i%4 for accumulator i.
// Here the MFMA M axis is the output feature (rows of S) and its N axis the
// token, so D is a tile of out^T; each lane stores 4 consecutive features of
// one token row as 8 bytes.
//
// Tiling: a workgroup computes BM features x BN tokens, waves WM x WN each,
// K in steps of 64 (dense) staged through LDS with a 2-stage double buffer and
// register prefetch of the next stage.  Rows beyond N or T are clamped on load
// and not stored; K beyond the end (K is a multiple of 16) is zero-filled.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "sp24_internal.hpp"

namespace sp24 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BK = 64;            // dense K per stage
constexpr int A_PAD = 8;          // halves of padding per LDS row
constexpr int S_LD = BK / 2 + A_PAD;   // compressed S row stride in LDS (halves)
constexpr int B_LD = BK + A_PAD;       // activation row stride in LDS (halves)

template <int BM, int BN, int WM, int WN>
struct SpmmCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int S_CHUNKS = BM * (BK / 2) / 8;   // 16-byte chunks of S per stage
  static constexpr int B_CHUNKS = BN * BK / 8;         // 16-byte chunks of A per stage
  static constexpr int S_PER_T = S_CHUNKS / THREADS;
  static constexpr int B_PER_T = B_CHUNKS / THREADS;
  static constexpr int M_PER_T = (BM * 4 + THREADS - 1) / THREADS;   // meta words per stage
  static_assert(S_CHUNKS % THREADS == 0 && B_CHUNKS % THREADS == 0, "tile/thread mismatch");
  static constexpr size_t SMEM = 2 * ((size_t)BM * S_LD * 2 + (size_t)BN * B_LD * 2 + (size_t)BM * 4 * 2);
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN)) void spmm_nt_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ vals, const uint16_t* __restrict__ meta,
    int64_t T, int64_t N, int64_t K, uint16_t* __restrict__ out, int tiles_m, int tiles_n) {
  using Cfg = SpmmCfg<BM, BN, WM, WN>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  _Float16* s_lds[2];
  _Float16* b_lds[2];
  uint16_t* m_lds[2];
  {
    unsigned char* p = smem_raw;
    for (int i = 0; i < 2; ++i) {
      s_lds[i] = reinterpret_cast<_Float16*>(p);
      p += (size_t)BM * S_LD * 2;
      b_lds[i] = reinterpret_cast<_Float16*>(p);
      p += (size_t)BN * B_LD * 2;
      m_lds[i] = reinterpret_cast<uint16_t*>(p);
      p += (size_t)BM * 4 * 2;
    }
  }

  // tile order: features fastest within a token panel, panels dealt so that
  // each XCD (8 of them, round-robin by workgroup id) works on nearby tiles
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int lin = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (lin >= ntiles) return;
  const int tn = lin / tiles_m, tm = lin - tn * tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % Cfg::WAVES_M, wn = wave / Cfg::WAVES_M;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t Kh = K / 2, Km = K / 16;
  const int nk = (int)((K + BK - 1) / BK);

  uint4 s_reg[Cfg::S_PER_T];
  uint4 b_reg[Cfg::B_PER_T];
  uint16_t m_reg[Cfg::M_PER_T];

  auto load_global = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < Cfg::S_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      const int row = c / (BK / 16), part = c % (BK / 16);
      const int64_t gr = min<int64_t>(m0 + row, N - 1);
      const int64_t kc = k0 / 2 + part * 8;
      s_reg[i] = kc < Kh ? *reinterpret_cast<const uint4*>(vals + gr * Kh + kc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      const int row = c / (BK / 8), part = c % (BK / 8);
      const int64_t gr = min<int64_t>(n0 + row, T - 1);
      const int64_t kc = k0 + part * 8;
      b_reg[i] = kc < K ? *reinterpret_cast<const uint4*>(A + gr * K + kc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::M_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      if (c < BM * 4) {
        const int row = c / 4, w = c % 4;
        const int64_t gr = min<int64_t>(m0 + row, N - 1);
        const int64_t kw = k0 / 16 + w;
        m_reg[i] = kw < Km ? meta[gr * Km + kw] : (uint16_t)0;
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::S_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      const int row = c / (BK / 16), part = c % (BK / 16);
      *reinterpret_cast<uint4*>(s_lds[buf] + row * S_LD + part * 8) = s_reg[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      const int row = c / (BK / 8), part = c % (BK / 8);
      *reinterpret_cast<uint4*>(b_lds[buf] + row * B_LD + part * 8) = b_reg[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::M_PER_T; ++i) {
      const int c = tid + i * Cfg::THREADS;
      if (c < BM * 4) m_lds[buf][c] = m_reg[i];
    }
  };

  f16v acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
    const _Float16* sl = s_lds[buf];
    const _Float16* bl = b_lds[buf];
    const uint16_t* ml = m_lds[buf];
    // meta words of this lane's rows: words g (k 0..31) and 2 + g (k 32..63)
    uint32_t idx[Cfg::TM][2];
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) {
      const int row = wm * WM + mt * 32 + l32;
      const uint2 mw = *reinterpret_cast<const uint2*>(ml + row * 4);
      idx[mt][0] = g ? (mw.x >> 16) : mw.x;
      idx[mt][1] = g ? (mw.y >> 16) : mw.y;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      h8 af[Cfg::TM];
      h16 bf[Cfg::TN];
#pragma unroll
      for (int mt = 0; mt < Cfg::TM; ++mt) {
        const int row = wm * WM + mt * 32 + l32;
        af[mt] = *reinterpret_cast<const h8*>(sl + row * S_LD + s * 16 + g * 8);
      }
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        const int row = wn * WN + nt * 32 + l32;
        const h8 lo = *reinterpret_cast<const h8*>(bl + row * B_LD + s * 32 + 8 * g);
        const h8 hi = *reinterpret_cast<const h8*>(bl + row * B_LD + s * 32 + 16 + 8 * g);
        bf[nt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
      for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
        for (int nt = 0; nt < Cfg::TN; ++nt)
          acc[mt][nt] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(af[mt], bf[nt], acc[mt][nt], (int)idx[mt][s], 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // epilogue: fp32 -> fp16 (round to nearest even), 4 features per 8-byte store
#pragma unroll
  for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
    for (int nt = 0; nt < Cfg::TN; ++nt) {
      const int64_t n = n0 + wn * WN + nt * 32 + l32;
      if (n >= T) continue;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int64_t m = m0 + wm * WM + mt * 32 + 8 * i4 + 4 * g;
        if (m >= N) continue;
        const f16v& a = acc[mt][nt];
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a[4 * i4 + 0]) |
                            (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a[4 * i4 + 1]) << 16;
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a[4 * i4 + 2]) |
                            (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a[4 * i4 + 3]) << 16;
        *reinterpret_cast<uint2*>(out + n * N + m) = make_uint2(lo, hi);
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T, int64_t N,
                      int64_t K, uint16_t* out, hipStream_t s) {
  using Cfg = SpmmCfg<BM, BN, WM, WN>;
  const int tiles_m = (int)((N + BM - 1) / BM), tiles_n = (int)((T + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  // thread-safe one-time opt-in to more than 64 KiB of dynamic LDS
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&spmm_nt_kernel<BM, BN, WM, WN>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((spmm_nt_kernel<BM, BN, WM, WN>), dim3(grid), dim3(Cfg::THREADS), Cfg::SMEM, s, A, vals, meta, T,
                     N, K, out, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm_nt(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T, int64_t N,
                          int64_t K, uint16_t* out, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  return launch_cfg<256, 128, 128, 64>(A, vals, meta, T, N, K, out, s);
}

}  // namespace sp24
