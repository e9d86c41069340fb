// Internal launch interface between the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace sp24 {

// Element offset of (r, c) in an n x m matrix stored in the compressed forms'
// blocked order: bands of 64 rows, each band's column blocks of width b
// (a power of two) stored one after the other, each block row-major; the
// last band and each band's last block may be narrower.  vals use b = 32
// halves (64 columns of W), meta b = 4 words.
__host__ __device__ inline int64_t form_off(int64_t r, int64_t c, int64_t n, int64_t m, int64_t b) {
  const int64_t r0 = r & ~(int64_t)63, c0 = c & ~(b - 1);
  const int64_t h = n - r0 < 64 ? n - r0 : 64, w = m - c0 < b ? m - c0 : b;
  return r0 * m + c0 * h + (r - r0) * w + (c - c0);
}
constexpr int64_t kValsBlock = 32, kMetaBlock = 4;

// Mask search only: idx[R/4][C/4].  R, C multiples of 4.
hipError_t launch_mask_search(const uint16_t* W, int64_t R, int64_t C, uint8_t* idx, hipStream_t s);

// One weight of a (batched) search+compress launch.
struct ScJob {
  const uint16_t* W;
  int64_t R, C;
  const uint8_t* idx_in;     // given masks (compress only), or nullptr to search
  uint8_t* idx_out;          // may be nullptr
  uint16_t* vals_row;        // (vals_row, meta_row) may both be nullptr
  uint16_t* meta_row;
  uint16_t* vals_col;        // (vals_col, meta_col) may both be nullptr
  uint16_t* meta_col;
  const uint8_t* idx_prev;   // previous masks (search only), or nullptr
  unsigned long long* flips; // receives += entries changed vs idx_prev; set iff idx_prev is
  int64_t tiles_c;           // filled in by the launcher
  int64_t tile_begin;        // filled in by the launcher
};
constexpr int kMaxScJobs = 8;
struct ScJobs {
  ScJob j[kMaxScJobs];
  int count;
  int64_t total_tiles;
  int cus;   // filled in by the launcher: the device's CU count
};
// Search (all jobs without idx_in) or compress with given masks (all jobs
// with idx_in); R, C multiples of 16.
hipError_t launch_search_compress_jobs(ScJobs jobs, bool search, hipStream_t s);

// Compression with either the searched masks (idx_in == nullptr: search and,
// if idx_out != nullptr, write idx) or given masks (idx_in != nullptr).
// R, C multiples of 16.  Either (vals, meta) pair may be null.
hipError_t launch_search_compress(const uint16_t* W, int64_t R, int64_t C, const uint8_t* idx_in,
                                  uint8_t* idx_out, uint16_t* vals_row, uint16_t* meta_row,
                                  uint16_t* vals_col, uint16_t* meta_col, hipStream_t s);

// *flips += number of mask entries that differ between the patterns
// a[0..n) and b[0..n) (indices >= 90 read as pattern 0).
hipError_t launch_flip_count(const uint8_t* a, const uint8_t* b, int64_t n, unsigned long long* flips,
                             hipStream_t s);

// dW[R][C] (fp32) = dY[T][R]^T X[T][C] + decay * (1 - M) * W, M from idx;
// W == nullptr leaves the decay term out.  R, C multiples of 16; T*R and T*C
// below 2^30.
hipError_t launch_weight_grad(const uint16_t* dY, const uint16_t* X, const uint16_t* W, const uint8_t* idx,
                              float decay, int64_t T, int64_t R, int64_t C, float* dW, hipStream_t s);

// GEGLU over U [T][2h] (blocks of `group` value columns, then `group` gate
// columns): out [T][h] = value * GELU(gate); the backward writes dU in U's
// layout.  h and group multiples of 8, h % group == 0.
hipError_t launch_geglu_fwd(const uint16_t* U, int64_t T, int64_t h, int64_t group, uint16_t* out, hipStream_t s);
hipError_t launch_geglu_bwd(const uint16_t* U, const uint16_t* dout, int64_t T, int64_t h, int64_t group,
                            uint16_t* dU, hipStream_t s);

// MVUE 2:4 estimate of M [rows][cols] (cols a multiple of 16) with one
// uniform U [rows][cols/4] per group, into the row form vals/meta (blocked
// order).
hipError_t launch_mvue(const uint16_t* M, const float* U, int64_t rows, int64_t cols, uint16_t* vals, uint16_t* meta,
                       hipStream_t s);

// out[T][N] = A[T][K] * S[N][K]^T with S in 2:4 row form along K:
// vals [N][K/2] fp16, meta [N][K/16], both in blocked order.  N, K multiples
// of 16.
hipError_t launch_spmm_nt(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T,
                          int64_t N, int64_t K, uint16_t* out, hipStream_t s);

// The same product with GEGLU fused into the epilogue: S's rows in blocks of
// 32 (16 value rows, then their 16 gate rows); gout[T][N/2] = value *
// GELU(gate) of the fp16 products.  out (the products, [T][N]) may be null
// when the fast path applies; otherwise hipErrorNotSupported.  N % 32 == 0.
hipError_t launch_spmm_nt_geglu(const uint16_t* A, const uint16_t* vals, const uint16_t* meta, int64_t T,
                                int64_t N, int64_t K, uint16_t* out, uint16_t* gout, hipStream_t s);

// One product of a grouped launch: out[T][N] = A[T][K] * S[N][K]^T.
struct GemmDesc {
  const uint16_t* A;
  const uint16_t* vals;
  const uint16_t* meta;
  uint16_t* out;
  int64_t T, N, K;
};
// Independent products in one persistent launch (fast-path shapes with
// K >= 192; the others run as single launches first).  work: 16 uint32 of
// device memory, zero on entry; a completed launch leaves them zero.
hipError_t launch_spmm_group(const GemmDesc* jobs, int count, unsigned int* work, hipStream_t s);
// The device address, on the current device, of the library's own copy of
// those 16 words (for the allocation-free entry point).
constexpr int kGroupScratchWords = 16;
hipError_t group_scratch(unsigned int** out);

}  // namespace sp24
