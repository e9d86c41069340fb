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

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "sp24_device.hpp"
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
      s_reg[i] = kc < Kh ? *reinterpret_cast<const uint4*>(vals + form_off(gr, kc, N, Kh, kValsBlock))
                         : make_uint4(0, 0, 0, 0);
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
        m_reg[i] = kw < Km ? meta[form_off(gr, kw, N, Km, kMetaBlock)] : (uint16_t)0;
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
  // opt-in to more than 64 KiB of dynamic LDS, once per device (the
  // attribute belongs to the current device's copy of the kernel)
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&spmm_nt_kernel<BM, BN, WM, WN>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    if (dev >= 0 && dev < 64) attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((spmm_nt_kernel<BM, BN, WM, WN>), dim3(grid), dim3(Cfg::THREADS), Cfg::SMEM, s, A, vals, meta, T,
                     N, K, out, tiles_m, tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fast path (K a multiple of 64, every operand below 2 GiB).
//
// Workgroup tile BM features x BN tokens in waves of WM x WN (launched as
// 256 x 256 with 8 waves of 128 x 64, two waves per SIMD).  A 3-stage LDS ring is filled by direct global->LDS buffer
// loads (no VGPR round trip), two stages ahead of the one being computed, so
// HBM/L2 latency hides behind two stages of MFMA work.  Rows past N or T read
// as zero (buffer bounds); they only feed outputs that are not stored.
//
// LDS layouts (per stage), both XOR-swizzled so that ds_read_b128 is free of
// bank conflicts for 8- and 16-lane groups:
//   S  [BM rows][4 chunks of 16 B]: chunk c of row r at slot c ^ fS(r)
//   B  [BN rows][8 chunks of 16 B]: chunk c of row r at slot c ^ fB(r)
//   meta [BM rows][2 dwords]
// A direct load writes 64 consecutive 16-byte LDS slots, one per lane, so each
// lane fetches the global chunk whose swizzled slot is its own lane index.

__device__ __forceinline__ int swz_s(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz_b(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BM, int BN, int WM, int WN>
struct FastCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int S_BYTES = BM * 64, B_BYTES = BN * 128, M_BYTES = BM * 8;
  static constexpr int S_LOADS = S_BYTES / 1024 / WAVES;   // 16-byte direct loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
  static constexpr int M_LOADS = M_BYTES / 256 / WAVES;    // 4-byte direct loads
  static constexpr int LOADS = S_LOADS + B_LOADS + M_LOADS;
  static_assert(S_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0 && M_BYTES % (256 * WAVES) == 0,
                "tile does not split evenly into direct loads");
  static_assert(LOADS <= 63, "vmcnt range");
};

// One BM x BN output tile at tile coordinates (tm, tn), computed by the
// whole workgroup with the ring in `smem`.  When `post` is set, thread 0
// stores `post_val` to *post_dst once the K loop is done, before the
// epilogue's stores (the grouped kernel hands its next tile index over
// there, while no load of this tile is still in flight).
template <int BM, int BN, int WM, int WN, bool kGeglu>
__device__ __forceinline__ void spmm_fast_tile(unsigned char* __restrict__ smem, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ vals, const uint16_t* __restrict__ meta,
                                               int64_t T, int64_t N, int64_t K, uint16_t* __restrict__ out,
                                               int64_t ldo, uint16_t* __restrict__ gout, int64_t ldg, int tm, int tn,
                                               int tid, bool post, int* post_dst, int post_val) {
  using Cfg = FastCfg<BM, BN, WM, WN>;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // the wave index is uniform across the wave; say so, since the direct
  // loads take their LDS destination from a scalar register
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WAVES_M, wn = wave / Cfg::WAVES_M;
  const int l32 = lane & 31, g = lane >> 5;
  const int nk = (int)(K / 64);

  // buffer resources based at this tile's first row; bytes past the matrix
  // end are out of range and load as zero.  S and meta are in blocked order:
  // a band of 64 rows starts every band_s (band_m) bytes, and stage kt of a
  // band of h rows is its contiguous block at kt * h * 64 (kt * h * 8) bytes.
  // Each load's rows (16 of S, 32 of meta) lie in one band, so its stage
  // stride st_s (st_m) is uniform across the wave: 4096 (512) for a full
  // band.  In the last band of an N % 64 != 0 operand, rows past N read bytes
  // of other rows or of nothing (zero); both only feed outputs that are not
  // stored.  Bands wholly past N start beyond the range.
  const i32x4 rs = make_rsrc(vals + m0 * (K / 2), (uint32_t)((N - m0) * K));
  const i32x4 rb = make_rsrc(A + n0 * K, (uint32_t)((T - n0) * K * 2));
  const i32x4 rm = make_rsrc(meta + m0 * (K / 16), (uint32_t)((N - m0) * (K / 8)));
  const int band_s = 64 * (int)K, band_m = 8 * (int)K;
  auto band_rows = [&](int band) {
    const int64_t left = N - m0 - 64 * band;
    return (int)(left >= 64 ? 64 : left > 0 ? left : 0);
  };
  int st_s[Cfg::S_LOADS], st_m[Cfg::M_LOADS];
#pragma unroll
  for (int i = 0; i < Cfg::S_LOADS; ++i) st_s[i] = band_rows((wave * Cfg::S_LOADS + i) / 4) * 64;
#pragma unroll
  for (int i = 0; i < Cfg::M_LOADS; ++i) st_m[i] = band_rows((wave * Cfg::M_LOADS + i) / 2) * 8;

  // per-lane global byte offsets of this wave's direct loads (stage 0)
  int off_s[Cfg::S_LOADS], off_b[Cfg::B_LOADS], off_m[Cfg::M_LOADS];
#pragma unroll
  for (int i = 0; i < Cfg::S_LOADS; ++i) {
    const int q = wave * Cfg::S_LOADS + i;          // 1 KiB: rows 16q .. 16q+15, contiguous in their block
    const int r = 16 * q + lane / 4, p = lane % 4;
    off_s[i] = (r / 64) * band_s + (r % 64) * 64 + ((p ^ swz_s(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_LOADS; ++i) {
    const int q = wave * Cfg::B_LOADS + i;          // rows 8q .. 8q+7
    const int r = 8 * q + lane / 8, p = lane % 8;
    off_b[i] = r * K * 2 + ((p ^ swz_b(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::M_LOADS; ++i) {
    const int q = wave * Cfg::M_LOADS + i;          // rows 32q .. 32q+31
    const int r = 32 * q + lane / 2;
    off_m[i] = (r / 64) * band_m + (r % 64) * 8 + (lane % 2) * 4;
  }

  // one of this wave's LOADS direct loads of stage kt (j in [0, LOADS))
  auto issue_one = [&](int j, int kt, unsigned char* sb, unsigned char* bb, unsigned char* mb) {
    if (j < Cfg::S_LOADS) {
      dma_b128(rs, lds_addr(sb) + (wave * Cfg::S_LOADS + j) * 1024, off_s[j] + kt * st_s[j]);
    } else if (j < Cfg::S_LOADS + Cfg::B_LOADS) {
      const int i = j - Cfg::S_LOADS;
      dma_b128(rb, lds_addr(bb) + (wave * Cfg::B_LOADS + i) * 1024, off_b[i] + kt * 128);
    } else {
      const int i = j - Cfg::S_LOADS - Cfg::B_LOADS;
      dma_b32(rm, lds_addr(mb) + (wave * Cfg::M_LOADS + i) * 256, off_m[i] + kt * st_m[i]);
    }
  };
  auto issue = [&](int kt, unsigned char* sb, unsigned char* bb, unsigned char* mb) {
    const int db = kt * 128;
#pragma unroll
    for (int i = 0; i < Cfg::S_LOADS; ++i)
      dma_b128(rs, lds_addr(sb) + (wave * Cfg::S_LOADS + i) * 1024, off_s[i] + kt * st_s[i]);
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i)
      dma_b128(rb, lds_addr(bb) + (wave * Cfg::B_LOADS + i) * 1024, off_b[i] + db);
#pragma unroll
    for (int i = 0; i < Cfg::M_LOADS; ++i)
      dma_b32(rm, lds_addr(mb) + (wave * Cfg::M_LOADS + i) * 256, off_m[i] + kt * st_m[i]);
  };

  // LDS read offsets of this lane (bytes), independent of the stage
  const int fs = swz_s(l32), fb = swz_b(l32);
  int rd_s[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) rd_s[st] = (wm * WM + l32) * 64 + (((2 * st + g) ^ fs) * 16);
  int rd_b[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int h = 0; h < 2; ++h) rd_b[st][h] = (wn * WN + l32) * 128 + (((4 * st + 2 * h + g) ^ fb) * 16);
  const int rd_m = (wm * WM + l32) * 8;

  f16v acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // register fragments of one K32 step
  struct Frags {
    h8 a[Cfg::TM];
    h16 b[Cfg::TN];
  };
  auto load_frags = [&](const unsigned char* sb, const unsigned char* bb, int st, Frags& f) {
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) f.a[mt] = *reinterpret_cast<const h8*>(sb + rd_s[st] + mt * 32 * 64);
#pragma unroll
    for (int nt = 0; nt < Cfg::TN; ++nt) {
      const h8 lo = *reinterpret_cast<const h8*>(bb + rd_b[st][0] + nt * 32 * 128);
      const h8 hi = *reinterpret_cast<const h8*>(bb + rd_b[st][1] + nt * 32 * 128);
      f.b[nt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
  };
  // meta words of this lane's rows for both K32 steps of a stage
  auto load_meta = [&](const unsigned char* mb, uint2 (&mw)[Cfg::TM]) {
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) mw[mt] = *reinterpret_cast<const uint2*>(mb + rd_m + mt * 32 * 8);
  };
  // The SMFMACs of one K32 step.  Two waves share each SIMD; raising the
  // priority of the wave in its MFMA block lets it issue back to back while
  // the other wave issues its LDS reads and direct loads in between.  When
  // kt_load >= 0, this wave's direct loads of stage kt_load go out one after
  // each SMFMAC rather than in a burst, so the texture unit drains steadily
  // and no wave stalls long on its in-order vector-memory issue.
  auto mfmas = [&](const Frags& f, const uint2 (&mw)[Cfg::TM], int st, int kt_load, unsigned char* sb,
                   unsigned char* bb, unsigned char* mb) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) {
      const uint32_t w = st ? mw[mt].y : mw[mt].x;
      const int idx = (int)(g ? (w >> 16) : w);
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        acc[mt][nt] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(f.a[mt], f.b[nt], acc[mt][nt], idx, 0, 0);
        const int j = mt * Cfg::TN + nt;
        if (j < Cfg::LOADS && kt_load >= 0) issue_one(j, kt_load, sb, bb, mb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = Cfg::TM * Cfg::TN; j < Cfg::LOADS; ++j)
      if (kt_load >= 0) issue_one(j, kt_load, sb, bb, mb);
    __builtin_amdgcn_s_setprio(0);
  };

  // vmcnt wait: allow `stages` stages of this wave's direct loads in flight
  auto wait_loads = [&](int stages) {
    // vmcnt in bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15 mean no wait
    if (stages >= 2) {
      constexpr int n = 2 * Cfg::LOADS;
      __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
    } else if (stages == 1) {
      constexpr int n = Cfg::LOADS;
      __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    }
  };

  unsigned char* const s_buf[3] = {smem, smem + Cfg::S_BYTES, smem + 2 * Cfg::S_BYTES};
  unsigned char* const b_buf[3] = {smem + 3 * Cfg::S_BYTES, smem + 3 * Cfg::S_BYTES + Cfg::B_BYTES,
                                   smem + 3 * Cfg::S_BYTES + 2 * Cfg::B_BYTES};
  unsigned char* const m_buf[3] = {smem + 3 * (Cfg::S_BYTES + Cfg::B_BYTES),
                                   smem + 3 * (Cfg::S_BYTES + Cfg::B_BYTES) + Cfg::M_BYTES,
                                   smem + 3 * (Cfg::S_BYTES + Cfg::B_BYTES) + 2 * Cfg::M_BYTES};

  // Pipeline.  Stage s (64 of K) is loaded into ring slot s % 3 three stages
  // ahead.  Within stage kt: the fragments of its second K32 step are read
  // while the first step's MFMAs run; then, mid-stage, the wave waits for
  // stage kt+1 to land, all waves meet at a barrier (after which nobody reads
  // slot kt % 3 again), stage kt+3 is issued into that slot, and the first
  // fragments of stage kt+1 are read while the second step's MFMAs run.
  for (int s = 0; s < 3; ++s)
    if (s < nk) issue(s, s_buf[s], b_buf[s], m_buf[s]);
  wait_loads(min(nk, 3) - 1);
  __builtin_amdgcn_s_barrier();
  Frags f0, f1;
  uint2 mw[Cfg::TM], mw_next[Cfg::TM];
  load_meta(m_buf[0], mw);
  load_frags(s_buf[0], b_buf[0], 0, f0);

  auto stage = [&](int kt, int cur, int nxt) {
    load_frags(s_buf[cur], b_buf[cur], 1, f1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0, mw, 0, -1, nullptr, nullptr, nullptr);
    __builtin_amdgcn_sched_barrier(0);
    wait_loads(kt + 2 < nk ? 1 : 0);
    // lgkmcnt(0): this wave's reads of slot kt % 3 are complete before the
    // barrier lets stage kt+3 overwrite it (vmcnt 63, expcnt 7 = no wait)
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < nk) {
      load_meta(m_buf[nxt], mw_next);
      load_frags(s_buf[nxt], b_buf[nxt], 0, f0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+3 goes into slot kt % 3, free since the barrier
    mfmas(f1, mw, 1, kt + 3 < nk ? kt + 3 : -1, s_buf[cur], b_buf[cur], m_buf[cur]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) mw[mt] = mw_next[mt];
  };
  for (int kt = 0; kt < nk; kt += 3) {
    stage(kt, 0, 1);
    if (kt + 1 < nk) stage(kt + 1, 1, 2);
    if (kt + 2 < nk) stage(kt + 2, 2, 0);
  }

  // Epilogue: fp32 -> fp16 (round to nearest even).  Each wave stages its
  // WN tokens x WM features in LDS (token-major, 16-byte chunks XOR-swizzled
  // by token) and writes whole contiguous token rows, so every store fills
  // complete cache lines.  The ring is idle now: all loads were waited for,
  // and the barrier makes sure no wave still reads its last fragments.
  static_assert(Cfg::WAVES * WN * WM * 2 <= 3 * (Cfg::S_BYTES + Cfg::B_BYTES), "staging does not fit");
  static_assert(WM == 128, "epilogue assumes 16 chunks of 8 features per token row");
  if (post) {
    // every wave takes the value through readfirstlane (wave 0 gets thread
    // 0's), so the wait for it is not on a divergent path and nothing is
    // left pending for the next tile's first instructions
    const int v = __builtin_amdgcn_readfirstlane(post_val);
    if (tid == 0) *post_dst = v;
  }
  __builtin_amdgcn_s_barrier();
  unsigned char* stage_base = smem + (size_t)wave * WN * WM * 2;
  auto h2 = [](float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) | (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y)
                                                                     << 16;
  };
  if constexpr (!kGeglu) {
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        const int t = nt * 32 + l32;                     // token within the wave tile
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f16v& a = acc[mt][nt];
          const uint32_t lo = h2(a[4 * i4 + 0], a[4 * i4 + 1]);
          const uint32_t hi = h2(a[4 * i4 + 2], a[4 * i4 + 3]);
          const int chunk = mt * 4 + i4;                 // 8 features per chunk: mt*32 + 8*i4 + 4g
          *reinterpret_cast<uint2*>(stage_base + t * 256 + ((chunk ^ (t & 15)) * 16) + 8 * g) = make_uint2(lo, hi);
        }
      }
    // the wave reads back only what it wrote, in order, so no barrier is needed
#pragma unroll 4
    for (int it = 0; it < WN * 16 / 64; ++it) {
      const int t = it * 4 + lane / 16, c = lane % 16;
      const uint4 v = *reinterpret_cast<const uint4*>(stage_base + t * 256 + ((c ^ (t & 15)) * 16));
      const int64_t n = n0 + wn * WN + t;
      const int64_t m = m0 + wm * WM + c * 8;
      if (n < T && m < N) *reinterpret_cast<uint4*>(out + n * ldo + m) = v;
    }
  } else {
    // The products are rounded to fp16 first (packed in pairs, which also
    // frees half the accumulator registers for the GELU arithmetic).
    uint32_t pk[Cfg::TM][Cfg::TN][8];
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt)
#pragma unroll
        for (int j = 0; j < 8; ++j) pk[mt][nt][j] = h2(acc[mt][nt][2 * j], acc[mt][nt][2 * j + 1]);
    if (out != nullptr) {
#pragma unroll
      for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
        for (int nt = 0; nt < Cfg::TN; ++nt) {
          const int t = nt * 32 + l32;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int chunk = mt * 4 + i4;
            *reinterpret_cast<uint2*>(stage_base + t * 256 + ((chunk ^ (t & 15)) * 16) + 8 * g) =
                make_uint2(pk[mt][nt][2 * i4], pk[mt][nt][2 * i4 + 1]);
          }
        }
#pragma unroll 4
      for (int it = 0; it < WN * 16 / 64; ++it) {
        const int t = it * 4 + lane / 16, c = lane % 16;
        const uint4 v = *reinterpret_cast<const uint4*>(stage_base + t * 256 + ((c ^ (t & 15)) * 16));
        const int64_t n = n0 + wn * WN + t;
        const int64_t m = m0 + wm * WM + c * 8;
        if (n < T && m < N) *reinterpret_cast<uint4*>(out + n * ldo + m) = v;
      }
      // this wave's reads of the staged products are back before the GEGLU
      // outputs overwrite them (lgkmcnt(0))
      __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    }
    // Accumulators 4*i4 + e (i4 < 2) and 4*(i4+2) + e of a 32-feature block
    // are features r and r + 16 of one token: a value and its gate.  The
    // WM/2 outputs per token are staged like the products (8 per chunk, chunk
    // index XOR-swizzled by token).
    auto half_of = [](uint32_t w, int hi) { return __builtin_bit_cast(_Float16, (uint16_t)(hi ? w >> 16 : w)); };
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        const int t = nt * 32 + l32;
#pragma unroll
        for (int i4 = 0; i4 < 2; ++i4) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (float)geglu_f16(half_of(pk[mt][nt][2 * i4 + e / 2], e & 1),
                                    half_of(pk[mt][nt][2 * (i4 + 2) + e / 2], e & 1));
          const int chunk = mt * 2 + i4;                 // outputs mt*16 + 8*i4 + 4g + e
          *reinterpret_cast<uint2*>(stage_base + t * 128 + ((chunk ^ (t & 7)) * 16) + 8 * g) =
              make_uint2(h2(o[0], o[1]), h2(o[2], o[3]));
        }
        // one 32 x 32 block at a time: keeping the GELU temporaries of
        // different blocks apart cut the epilogue's register spills (132 -> 96
        // bytes per lane) and 2-4 us per 6400 x 1600 call, same outputs
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll 4
    for (int it = 0; it < WN * 8 / 64; ++it) {
      const int t = it * 8 + lane / 8, c = lane % 8;
      const uint4 v = *reinterpret_cast<const uint4*>(stage_base + t * 128 + ((c ^ (t & 7)) * 16));
      const int64_t n = n0 + wn * WN + t;
      const int64_t m = (m0 + wm * WM) / 2 + c * 8;
      if (n < T && m < N / 2) *reinterpret_cast<uint4*>(gout + n * ldg + m) = v;
    }
  }
}

// kGeglu: the feature rows of S come in blocks of 32, 16 value rows then the
// 16 matching gate rows, and the epilogue also writes gout[T][ldg] columns
// [0, N/2) = value * GELU(gate) from the fp16-rounded products, with the
// GEGLU kernel's GELU code.  `out` may then be null (the products are not
// stored).
template <int BM, int BN, int WM, int WN, bool kGeglu>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN), 1) void spmm_nt_fast_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ vals, const uint16_t* __restrict__ meta,
    int64_t T, int64_t N, int64_t K, uint16_t* __restrict__ out, int64_t ldo, uint16_t* __restrict__ gout,
    int64_t ldg, int tiles_m, int tiles_n) {
  using Cfg = FastCfg<BM, BN, WM, WN>;
  // one LDS block: 3 S slots, 3 B slots, 3 meta slots (the epilogue reuses
  // the start of it to stage the output tile)
  __shared__ __align__(1024) unsigned char smem[3 * (Cfg::S_BYTES + Cfg::B_BYTES + Cfg::M_BYTES)];

  // tile order: groups of kGroupM feature tiles, token tiles within a group,
  // features fastest; each XCD (workgroups are dealt round-robin to 8 XCDs)
  // takes a contiguous run of that order so concurrent tiles share operands in
  // its L2
  constexpr int kGroupM = 8;
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int lin = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (lin >= ntiles) return;
  const int group = lin / (kGroupM * tiles_n);
  const int gm0 = group * kGroupM;
  const int gsize = min(kGroupM, tiles_m - gm0);
  const int in_group = lin - group * kGroupM * tiles_n;
  // the tile indices are uniform; readfirstlane keeps them (and the buffer
  // descriptors built from them) in scalar registers
  const int tn = __builtin_amdgcn_readfirstlane(in_group / gsize);
  const int tm = __builtin_amdgcn_readfirstlane(gm0 + in_group % gsize);
  spmm_fast_tile<BM, BN, WM, WN, kGeglu>(smem, A, vals, meta, T, N, K, out, ldo, gout, ldg, tm, tn,
                                         (int)threadIdx.x, false, nullptr, 0);
}

// ---------------------------------------------------------------------------
// Grouped launch: several independent fast-path GEMMs (the forward and
// input-gradient products of both FFN linears, say) in one persistent launch.
//
// One workgroup per CU loops over tiles.  The tiles of every job are split
// into 8 contiguous runs of the single launch's tile order (groups of 8
// feature tiles, token tiles within a group, features fastest), one per XCD,
// and queue x lists run x of each job, jobs in the order given (the host puts
// the longest reductions first).  Workgroup b serves queue b % 8 (the XCD it
// is dispatched to), taking the next tile with one atomic increment, so the
// concurrent tiles of an XCD share operand strips in its L2, and tiles of
// different lengths pack the CUs with no partial round per GEMM.  Each
// workgroup takes its next tile index while the current tile runs and hands
// it over in LDS once the tile's K loop is done.
//
// work[0..7] are the queue heads and work[8..15] count the workgroups that
// found their queue empty; the last one of a queue sets both back to zero,
// so a launch that runs to completion leaves the workspace as it found it
// (all zero).
constexpr int kMaxGroupJobs = 8;
struct GroupJob {
  const uint16_t* A;
  const uint16_t* vals;
  const uint16_t* meta;
  uint16_t* out;
  int64_t T, N, K;
  int tiles_m, tiles_n;
};
struct GroupArgs {
  GroupJob job[kMaxGroupJobs];
  int njobs;
  int lo[8][kMaxGroupJobs];    // first position of queue x's run in job j's tile order
  int cnt[8][kMaxGroupJobs];   // tiles of job j in queue x
  int total[8];                // tiles in queue x
  int wgs[8];                  // workgroups serving queue x
};

// LDS-only workgroup barrier: this wave's LDS accesses are complete, and the
// compiler moves no memory access across it (no wait for global stores).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN), 1) void spmm_group_kernel(GroupArgs args,
                                                                                   unsigned int* __restrict__ work) {
  using Cfg = FastCfg<BM, BN, WM, WN>;
  __shared__ __align__(1024) unsigned char smem[3 * (Cfg::S_BYTES + Cfg::B_BYTES + Cfg::M_BYTES)];
  __shared__ int sh_next;
  constexpr int kGroupM = 8;
  const int x = (int)(blockIdx.x % 8);
  unsigned int* const queue = work + x;
  unsigned int* const done = work + 8 + x;
  const int total = args.total[x];
  if (threadIdx.x == 0) sh_next = (int)atomicAdd(queue, 1u);
  lds_barrier();
  int cur = __builtin_amdgcn_readfirstlane(sh_next);
  while (cur < total) {
    // the tile after this one, taken now and handed over after the K loop
    int nxt;   // only thread 0's value is used; no initialisation to wait behind
    if (threadIdx.x == 0) {
      // the address goes through a vector register, so the compiler cannot
      // turn this into a wave-aggregated atomic whose result it waits for at
      // once: the value is first needed after the K loop
      typedef __attribute__((address_space(1))) unsigned int global_u32;
      global_u32* q = (global_u32*)queue;
      asm volatile("" : "+v"(q));
      nxt = (int)__hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int j = 0, i = cur;
    while (j + 1 < args.njobs && i >= args.cnt[x][j]) {
      i -= args.cnt[x][j];
      ++j;
    }
    const GroupJob& jb = args.job[j];
    const int tiles_m = jb.tiles_m, tiles_n = jb.tiles_n;
    const int lin = args.lo[x][j] + i;
    const int group = lin / (kGroupM * tiles_n);
    const int gm0 = group * kGroupM;
    const int gsize = min(kGroupM, tiles_m - gm0);
    const int in_group = lin - group * kGroupM * tiles_n;
    const int tn = __builtin_amdgcn_readfirstlane(in_group / gsize);
    const int tm = __builtin_amdgcn_readfirstlane(gm0 + in_group % gsize);
    // the thread index through an opaque copy, so that the tile's per-lane
    // offsets are recomputed for every tile rather than hoisted out of this
    // loop (held across it they would not fit in the registers)
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    spmm_fast_tile<BM, BN, WM, WN, false>(smem, jb.A, jb.vals, jb.meta, jb.T, jb.N, jb.K, jb.out, jb.N, nullptr, 0,
                                          tm, tn, tid, true, &sh_next, nxt);
    // every wave has read back its staged outputs (the ring is free for the
    // next tile's loads) and the next index is visible
    lds_barrier();
    cur = __builtin_amdgcn_readfirstlane(sh_next);
  }
  if (threadIdx.x == 0) {
    // this workgroup's last increment of the queue has returned (its value
    // ended the loop); the last workgroup of the queue resets it
    const unsigned int d = atomicAdd(done, 1u);
    if (d == (unsigned int)args.wgs[x] - 1u) {
      atomicExch(queue, 0u);
      atomicExch(done, 0u);
    }
  }
}

// out[T][ldo] columns [0, N) = A * S^T for the N feature rows of S given;
// with kGeglu also gout[T][ldg] columns [0, N/2).
template <int BM, int BN, int WM, int WN, bool kGeglu = false>
hipError_t launch_fast(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T, int64_t N,
                       int64_t K, uint16_t* out, int64_t ldo, hipStream_t s, uint16_t* gout = nullptr,
                       int64_t ldg = 0) {
  using Cfg = FastCfg<BM, BN, WM, WN>;
  const int tiles_m = (int)((N + BM - 1) / BM), tiles_n = (int)((T + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  hipLaunchKernelGGL((spmm_nt_fast_kernel<BM, BN, WM, WN, kGeglu>), dim3(grid), dim3(Cfg::THREADS), 0, s, A, vals,
                     meta, T, N, K, out, ldo, gout, ldg, tiles_m, tiles_n);
  return hipGetLastError();
}

bool fast_path(int64_t T, int64_t N, int64_t K) {
  // Buffer offsets are 32-bit.  A tile computes r * K * 2 for each of its
  // 256 rows, also rows past T or N (whose loads are out of range), so the
  // bound is on 256 rows of K, not only on the matrices.
  constexpr int64_t kMaxBuf = (int64_t)1 << 31;
  return K % 64 == 0 && K > 0 && K * 512 < kMaxBuf && T * K * 2 < kMaxBuf && N * K < kMaxBuf &&
         T * N * 2 < ((int64_t)1 << 40);
}

// The last strip of w <= 256 features after a split runs as 128 x 128 tiles
// when it is wider than 128 features, else as 256 x 64 tiles (128 x 128
// tiles of a narrow strip would leave half the CUs idle).  Both shapes keep
// four waves of 128 x 32 per CU.  The 128 x 128 tile touches a third fewer
// cache lines per stage than 256 x 64, whose 256 rows of S and of meta serve
// a quarter of a full tile's work (1.5B shapes: 243 -> 236 us per
// 6400-feature GEMM, bit-identical).
bool wide_tail(int64_t w) { return w > 128; }
int64_t tail_tiles(int64_t T, int64_t w) { return wide_tail(w) ? 2 * ((T + 127) / 128) : (T + 63) / 64; }

// The feature rows that fill whole rounds of 256 x 256 tiles on the device,
// when the remaining strip is better run as smaller tiles in one partial
// round (see launch_spmm_nt); 0 when no split pays.
int64_t split_features(int64_t T, int64_t N) {
  const int64_t cus = device_cu_count();
  const int64_t tiles_n = (T + 255) / 256, tiles_m = (N + 255) / 256;
  if (tiles_m < 2 || (tiles_m * tiles_n) % cus == 0 || ((tiles_m - 1) * tiles_n) % cus != 0) return 0;
  const int64_t n1 = (tiles_m - 1) * 256;
  return tail_tiles(T, N - n1) <= cus ? n1 : 0;
}

}  // namespace

hipError_t launch_spmm_nt(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T, int64_t N,
                          int64_t K, uint16_t* out, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  if (fast_path(T, N, K)) {
    // 256 x 256 tiles, 8 waves (two per SIMD) of 128 features x 64 tokens.
    // When the tile count leaves a last, partly filled round of workgroups,
    // the leading feature tiles that fill whole rounds run first and the last
    // strip (up to 256 features) runs as tiles with a quarter of the work
    // each (split_features), so the tail takes a fraction of a round.
    const int64_t n1 = split_features(T, N);
    if (n1 > 0) {
      hipError_t e = launch_fast<256, 256, 128, 64>(A, vals, meta, T, n1, K, out, N, s);
      if (e != hipSuccess) return e;
      const uint16_t* v2 = vals + n1 * (K / 2);
      const uint16_t* m2 = meta + n1 * (K / 16);
      if (wide_tail(N - n1)) return launch_fast<128, 128, 128, 32>(A, v2, m2, T, N - n1, K, out + n1, N, s);
      return launch_fast<256, 64, 128, 32>(A, v2, m2, T, N - n1, K, out + n1, N, s);
    }
    return launch_fast<256, 256, 128, 64>(A, vals, meta, T, N, K, out, N, s);
  }
  return launch_cfg<256, 128, 128, 64>(A, vals, meta, T, N, K, out, s);
}

hipError_t launch_spmm_nt_geglu(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T, int64_t N,
                                int64_t K, uint16_t* out, uint16_t* gout, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  if (!fast_path(T, N, K)) {
    // the products must be stored to apply GEGLU afterwards
    if (out == nullptr) return hipErrorNotSupported;
    const hipError_t e = launch_spmm_nt(A, vals, meta, T, N, K, out, s);
    if (e != hipSuccess) return e;
    return launch_geglu_fwd(out, T, N / 2, 16, gout, s);
  }
  const int64_t n1 = split_features(T, N);
  if (n1 > 0) {
    hipError_t e = launch_fast<256, 256, 128, 64, true>(A, vals, meta, T, n1, K, out, N, s, gout, N / 2);
    if (e != hipSuccess) return e;
    const uint16_t* v2 = vals + n1 * (K / 2);
    const uint16_t* m2 = meta + n1 * (K / 16);
    uint16_t* o2 = out ? out + n1 : nullptr;
    if (wide_tail(N - n1))
      return launch_fast<128, 128, 128, 32, true>(A, v2, m2, T, N - n1, K, o2, N, s, gout + n1 / 2, N / 2);
    return launch_fast<256, 64, 128, 32, true>(A, v2, m2, T, N - n1, K, o2, N, s, gout + n1 / 2, N / 2);
  }
  return launch_fast<256, 256, 128, 64, true>(A, vals, meta, T, N, K, out, N, s, gout, N / 2);
}

// The grouped launch's queue counters for callers that cannot allocate: 16
// words of device memory in the library itself, one copy per GPU (zero when
// the library is loaded, and left zero by every launch that completes).  Host
// code must not pass the array's name to a kernel: it stands for a host-side
// symbol.  Its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current.
static __device__ __align__(256) unsigned int scratch[kGroupScratchWords];

hipError_t group_scratch(unsigned int** out) {
  static std::atomic<unsigned int*> ptrs[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned int* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_spmm_group(const GemmDesc* jobs, int count, unsigned int* work, hipStream_t s) {
  // jobs the fast kernel cannot take run as single launches first
  GroupArgs args{};
  int order[kMaxGroupJobs];
  int n = 0;
  for (int j = 0; j < count; ++j) {
    const GemmDesc& g = jobs[j];
    if (g.T == 0 || g.N == 0) continue;
    if (!fast_path(g.T, g.N, g.K) || g.K < 3 * 64 || n == kMaxGroupJobs) {
      const hipError_t e = launch_spmm_nt(g.A, g.vals, g.meta, g.T, g.N, g.K, g.out, s);
      if (e != hipSuccess) return e;
      continue;
    }
    order[n++] = j;
  }
  if (n == 0) return hipSuccess;
  // longest reductions first: their tiles take the most time, and the short
  // ones then fill in behind them
  for (int a = 1; a < n; ++a)
    for (int b = a; b > 0 && jobs[order[b]].K > jobs[order[b - 1]].K; --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  int64_t all_tiles = 0;
  args.njobs = n;
  for (int q = 0; q < n; ++q) {
    const GemmDesc& g = jobs[order[q]];
    GroupJob& jb = args.job[q];
    jb.A = g.A;
    jb.vals = g.vals;
    jb.meta = g.meta;
    jb.out = g.out;
    jb.T = g.T;
    jb.N = g.N;
    jb.K = g.K;
    jb.tiles_m = (int)((g.N + 255) / 256);
    jb.tiles_n = (int)((g.T + 255) / 256);
    const int64_t ntiles = (int64_t)jb.tiles_m * jb.tiles_n;
    all_tiles += ntiles;
    for (int x = 0; x < 8; ++x) {
      const int64_t lo = x * ntiles / 8, hi = (x + 1) * ntiles / 8;
      args.lo[x][q] = (int)lo;
      args.cnt[x][q] = (int)(hi - lo);
      args.total[x] += (int)(hi - lo);
    }
  }
  // one workgroup per CU (the ring takes 150 KB of LDS), a multiple of 8 so
  // every queue has the same number of workgroups, and no more than there
  // are tiles
  int64_t grid = device_cu_count();
  grid = std::min<int64_t>(grid, (all_tiles + 7) / 8 * 8);
  grid = std::max<int64_t>(8, grid / 8 * 8);
  for (int x = 0; x < 8; ++x) args.wgs[x] = (int)(grid / 8);
  using Cfg = FastCfg<256, 256, 128, 64>;
  hipLaunchKernelGGL((spmm_group_kernel<256, 256, 128, 64>), dim3((unsigned)grid), dim3(Cfg::THREADS), 0, s, args,
                     work);
  return hipGetLastError();
}

}  // namespace sp24
