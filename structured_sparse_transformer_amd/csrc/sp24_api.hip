// C ABI of the transposable 2:4 FFN kernels (declared in include/sp24.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues its kernels on the caller's stream and returns.  Nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "sp24.h"
#include "sp24_internal.hpp"
#include "sp24_patterns.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;        // each dimension below 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 40;      // each matrix below 2^40 entries
// the streaming kernels (GEGLU, MVUE) launch one work-item per 8 or 16
// entries in one grid dimension, whose work-items HIP counts in 32 bits:
// 256-wide workgroups allow at most 2^32 - 256 of them
constexpr int64_t kMaxLaunchItems = ((int64_t)1 << 32) - 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

int check_dims(int64_t a, int64_t b, int64_t mult) {
  if (a < 0 || b < 0 || a % mult != 0 || b % mult != 0) return SP24_ERR_SHAPE;
  if (a >= kMaxDim || b >= kMaxDim) return SP24_ERR_TOO_LARGE;
  if (a != 0 && b >= kMaxElems / a) return SP24_ERR_TOO_LARGE;
  return SP24_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? SP24_OK : SP24_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_pair(const void* vals, const void* meta, bool& present) {
  present = vals != nullptr || meta != nullptr;
  if (present && (vals == nullptr || meta == nullptr)) return SP24_ERR_NULL;
  if (present && (!aligned16(vals) || !aligned16(meta))) return SP24_ERR_ALIGN;
  return SP24_OK;
}

// Validates one search/compress job (shared by the single and batched calls).
int check_compress(const void* W, const uint8_t* idx_in, uint8_t* idx_out, int64_t R, int64_t C, void* vals_row,
                   uint16_t* meta_row, void* vals_col, uint16_t* meta_col) {
  int st = check_dims(R, C, 16);
  if (st != SP24_OK) return st;
  bool has_row = false, has_col = false;
  if ((st = check_pair(vals_row, meta_row, has_row)) != SP24_OK) return st;
  if ((st = check_pair(vals_col, meta_col, has_col)) != SP24_OK) return st;
  if (!has_row && !has_col) return SP24_ERR_NULL;
  if (R == 0 || C == 0) return SP24_OK;
  if (W == nullptr) return SP24_ERR_NULL;
  if (!aligned16(W) || (idx_in && !aligned16(idx_in)) || (idx_out && !aligned16(idx_out))) return SP24_ERR_ALIGN;
  return SP24_OK;
}

int compress_common(const void* W, const uint8_t* idx_in, uint8_t* idx_out, int64_t R, int64_t C, void* vals_row,
                    uint16_t* meta_row, void* vals_col, uint16_t* meta_col, void* stream) {
  const int st = check_compress(W, idx_in, idx_out, R, C, vals_row, meta_row, vals_col, meta_col);
  if (st != SP24_OK || R == 0 || C == 0) return st;
  return launch_status(sp24::launch_search_compress(
      static_cast<const uint16_t*>(W), R, C, idx_in, idx_out, static_cast<uint16_t*>(vals_row), meta_row,
      static_cast<uint16_t*>(vals_col), meta_col, as_stream(stream)));
}

int check_spmm(const void* A, const void* vals, const uint16_t* meta, int64_t T, int64_t N, int64_t K,
               const void* out) {
  if (T < 0) return SP24_ERR_SHAPE;
  int st = check_dims(N, K, 16);
  if (st != SP24_OK) return st;
  if (T >= kMaxDim) return SP24_ERR_TOO_LARGE;
  if (T != 0 && (K >= kMaxElems / T || N >= kMaxElems / T)) return SP24_ERR_TOO_LARGE;
  if (T == 0 || N == 0) return SP24_OK;
  if (out == nullptr || (K != 0 && (A == nullptr || vals == nullptr || meta == nullptr))) return SP24_ERR_NULL;
  if (!aligned16(out) || (K != 0 && (!aligned16(A) || !aligned16(vals) || !aligned16(meta)))) return SP24_ERR_ALIGN;
  return SP24_OK;
}

int spmm_common(const void* A, const void* vals, const uint16_t* meta, int64_t T, int64_t N, int64_t K, void* out,
                void* stream) {
  const int st = check_spmm(A, vals, meta, T, N, K, out);
  if (st != SP24_OK || T == 0 || N == 0) return st;
  return launch_status(sp24::launch_spmm_nt(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(vals), meta,
                                            T, N, K, static_cast<uint16_t*>(out), as_stream(stream)));
}

int check_geglu(int64_t T, int64_t h, int64_t group) {
  if (T < 0 || h < 0 || group <= 0 || h % 8 != 0 || group % 8 != 0 || (h != 0 && h % group != 0))
    return SP24_ERR_SHAPE;
  if (T >= kMaxDim || h >= kMaxDim || (T != 0 && 2 * h >= kMaxElems / T)) return SP24_ERR_TOO_LARGE;
  if (T != 0 && h / 8 > kMaxLaunchItems / T) return SP24_ERR_TOO_LARGE;   // T * h/8 work-items
  return SP24_OK;
}

}  // namespace

extern "C" {

int sp24_mask_search(const void* W, int64_t R, int64_t C, uint8_t* idx, void* stream) {
  int st = check_dims(R, C, 4);
  if (st != SP24_OK) return st;
  if (R == 0 || C == 0) return SP24_OK;
  if (W == nullptr || idx == nullptr) return SP24_ERR_NULL;
  if (!aligned16(W) || !aligned16(idx)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_mask_search(static_cast<const uint16_t*>(W), R, C, idx, as_stream(stream)));
}

int sp24_compress(const void* W, const uint8_t* idx, int64_t R, int64_t C, void* vals_row, uint16_t* meta_row,
                  void* vals_col, uint16_t* meta_col, void* stream) {
  if (idx == nullptr && R > 0 && C > 0 && R % 16 == 0 && C % 16 == 0) return SP24_ERR_NULL;
  return compress_common(W, idx, nullptr, R, C, vals_row, meta_row, vals_col, meta_col, stream);
}

int sp24_search_compress(const void* W, int64_t R, int64_t C, uint8_t* idx, void* vals_row, uint16_t* meta_row,
                         void* vals_col, uint16_t* meta_col, void* stream) {
  return compress_common(W, nullptr, idx, R, C, vals_row, meta_row, vals_col, meta_col, stream);
}

int sp24_search_compress_batch(const sp24_sc_job* jobs, int count, void* stream) {
  if (jobs == nullptr) return SP24_ERR_NULL;
  if (count < 1 || count > SP24_MAX_BATCH || count > sp24::kMaxScJobs) return SP24_ERR_SHAPE;
  sp24::ScJobs batch{};
  for (int k = 0; k < count; ++k) {
    const sp24_sc_job& j = jobs[k];
    const int st = check_compress(j.W, nullptr, j.idx, j.R, j.C, j.vals_row, j.meta_row, j.vals_col, j.meta_col);
    if (st != SP24_OK) return st;
    if ((j.idx_prev == nullptr) != (j.flips == nullptr)) return SP24_ERR_NULL;
    if (j.R == 0 || j.C == 0) continue;
    if (j.flips && (!aligned16(j.idx_prev) || !aligned8(j.flips))) return SP24_ERR_ALIGN;
    batch.j[batch.count++] = sp24::ScJob{static_cast<const uint16_t*>(j.W), j.R, j.C, nullptr, j.idx,
                                         static_cast<uint16_t*>(j.vals_row), j.meta_row,
                                         static_cast<uint16_t*>(j.vals_col), j.meta_col, j.idx_prev,
                                         reinterpret_cast<unsigned long long*>(j.flips), 0, 0};
  }
  if (batch.count == 0) return SP24_OK;
  return launch_status(sp24::launch_search_compress_jobs(batch, true, as_stream(stream)));
}

int sp24_flip_count(const uint8_t* idx_prev, const uint8_t* idx_new, int64_t nblocks, uint64_t* flips,
                    void* stream) {
  if (nblocks < 0) return SP24_ERR_SHAPE;
  if (nblocks >= kMaxElems) return SP24_ERR_TOO_LARGE;
  if (nblocks == 0) return SP24_OK;
  if (idx_prev == nullptr || idx_new == nullptr || flips == nullptr) return SP24_ERR_NULL;
  if (!aligned16(idx_prev) || !aligned16(idx_new) || !aligned8(flips)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_flip_count(idx_prev, idx_new, nblocks,
                                               reinterpret_cast<unsigned long long*>(flips), as_stream(stream)));
}

int sp24_spmm_fwd(const void* X, const void* vals_row, const uint16_t* meta_row, int64_t T, int64_t R, int64_t C,
                  void* Y, void* stream) {
  // Y[T][R] = X[T][C] * Ws^T: output features R, reduction over C
  return spmm_common(X, vals_row, meta_row, T, R, C, Y, stream);
}

int sp24_spmm_fwd_geglu(const void* X, const void* vals_row, const uint16_t* meta_row, int64_t T, int64_t R,
                        int64_t C, void* U, void* out, void* stream) {
  if (T < 0) return SP24_ERR_SHAPE;
  int st = check_dims(R, C, 16);
  if (st != SP24_OK) return st;
  if (R % 32 != 0) return SP24_ERR_SHAPE;
  if (T >= kMaxDim) return SP24_ERR_TOO_LARGE;
  if (T != 0 && (C >= kMaxElems / T || R >= kMaxElems / T)) return SP24_ERR_TOO_LARGE;
  // the GEGLU kernel that finishes the shapes the fused kernel does not take
  if (T != 0 && R / 16 > kMaxLaunchItems / T) return SP24_ERR_TOO_LARGE;
  if (T == 0 || R == 0) return SP24_OK;
  if (out == nullptr || (C != 0 && (X == nullptr || vals_row == nullptr || meta_row == nullptr))) return SP24_ERR_NULL;
  if (!aligned16(out) || (U && !aligned16(U)) ||
      (C != 0 && (!aligned16(X) || !aligned16(vals_row) || !aligned16(meta_row))))
    return SP24_ERR_ALIGN;
  const hipError_t e = sp24::launch_spmm_nt_geglu(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(vals_row),
                                                  meta_row, T, R, C, static_cast<uint16_t*>(U),
                                                  static_cast<uint16_t*>(out), as_stream(stream));
  if (e == hipErrorNotSupported) return SP24_ERR_UNSUPPORTED;
  return launch_status(e);
}

// Checks a group's products and fills the launcher's descriptors.
int check_group(const sp24_gemm* gemms, int count, sp24::GemmDesc* d) {
  if (gemms == nullptr) return SP24_ERR_NULL;
  if (count < 1 || count > SP24_MAX_GROUP) return SP24_ERR_SHAPE;
  for (int j = 0; j < count; ++j) {
    const sp24_gemm& g = gemms[j];
    const int st = check_spmm(g.A, g.vals, g.meta, g.T, g.N, g.K, g.out);
    if (st != SP24_OK) return st;
    d[j] = {static_cast<const uint16_t*>(g.A), static_cast<const uint16_t*>(g.vals), g.meta,
            static_cast<uint16_t*>(g.out), g.T, g.N, g.K};
  }
  return SP24_OK;
}

int sp24_spmm_group(const sp24_gemm* gemms, int count, void* workspace, void* stream) {
  static_assert(SP24_MAX_GROUP <= 8, "the launcher's job table holds 8 products");
  static_assert(SP24_GROUP_WORKSPACE_BYTES == 4 * sp24::kGroupScratchWords, "workspace size");
  sp24::GemmDesc d[SP24_MAX_GROUP];
  const int st = check_group(gemms, count, d);
  if (st != SP24_OK) return st;
  if (workspace == nullptr) return SP24_ERR_NULL;
  if (!aligned16(workspace)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_spmm_group(d, count, static_cast<unsigned int*>(workspace), as_stream(stream)));
}

int sp24_spmm_group_noalloc(const sp24_gemm* gemms, int count, void* stream) {
  sp24::GemmDesc d[SP24_MAX_GROUP];
  const int st = check_group(gemms, count, d);
  if (st != SP24_OK) return st;
  unsigned int* work = nullptr;
  if (sp24::group_scratch(&work) != hipSuccess) return SP24_ERR_LAUNCH;
  return launch_status(sp24::launch_spmm_group(d, count, work, as_stream(stream)));
}

int sp24_spmm_bwd_input(const void* dY, const void* vals_col, const uint16_t* meta_col, int64_t T, int64_t R,
                        int64_t C, void* dX, void* stream) {
  // dX[T][C] = dY[T][R] * Ws: output features C, reduction over R
  return spmm_common(dY, vals_col, meta_col, T, C, R, dX, stream);
}

int sp24_weight_grad(const void* dY, const void* X, const void* W, const uint8_t* idx, float decay, int64_t T,
                     int64_t R, int64_t C, float* dW, void* stream) {
  if (T < 0) return SP24_ERR_SHAPE;
  int st = check_dims(R, C, 16);
  if (st != SP24_OK) return st;
  if (T >= kMaxDim) return SP24_ERR_TOO_LARGE;
  // token-row offsets of the direct loads are 32-bit byte offsets
  if (T != 0 && (R >= ((int64_t)1 << 30) / T || C >= ((int64_t)1 << 30) / T)) return SP24_ERR_TOO_LARGE;
  if ((W == nullptr) != (idx == nullptr)) return SP24_ERR_NULL;
  if (R == 0 || C == 0) return SP24_OK;
  if (dW == nullptr || (T != 0 && (dY == nullptr || X == nullptr))) return SP24_ERR_NULL;
  if (!aligned16(dW) || (T != 0 && (!aligned16(dY) || !aligned16(X))) || (W && (!aligned16(W) || !aligned16(idx))))
    return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_weight_grad(static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(X),
                                                static_cast<const uint16_t*>(W), idx, decay, T, R, C, dW,
                                                as_stream(stream)));
}

int sp24_geglu_fwd(const void* U, int64_t T, int64_t h, int64_t group, void* out, void* stream) {
  const int st = check_geglu(T, h, group);
  if (st != SP24_OK || T == 0 || h == 0) return st;
  if (U == nullptr || out == nullptr) return SP24_ERR_NULL;
  if (!aligned16(U) || !aligned16(out)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_geglu_fwd(static_cast<const uint16_t*>(U), T, h, group,
                                              static_cast<uint16_t*>(out), as_stream(stream)));
}

int sp24_geglu_bwd(const void* U, const void* dout, int64_t T, int64_t h, int64_t group, void* dU, void* stream) {
  const int st = check_geglu(T, h, group);
  if (st != SP24_OK || T == 0 || h == 0) return st;
  if (U == nullptr || dout == nullptr || dU == nullptr) return SP24_ERR_NULL;
  if (!aligned16(U) || !aligned16(dout) || !aligned16(dU)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_geglu_bwd(static_cast<const uint16_t*>(U), static_cast<const uint16_t*>(dout), T,
                                              h, group, static_cast<uint16_t*>(dU), as_stream(stream)));
}

int sp24_mvue(const void* M, const float* U, int64_t rows, int64_t cols, void* vals, uint16_t* meta, void* stream) {
  int st = check_dims(rows, cols, 1);
  if (st != SP24_OK) return st;
  if (cols % 16 != 0) return SP24_ERR_SHAPE;
  // one workgroup of 256 per 64 x 256 region (four column blocks of a 64-row band)
  if (((rows + 63) / 64) * ((cols / 16 + 15) / 16) > kMaxLaunchItems / 256) return SP24_ERR_TOO_LARGE;
  if (rows == 0 || cols == 0) return SP24_OK;
  if (M == nullptr || U == nullptr || vals == nullptr || meta == nullptr) return SP24_ERR_NULL;
  if (!aligned16(M) || !aligned16(U) || !aligned16(vals) || !aligned16(meta)) return SP24_ERR_ALIGN;
  return launch_status(sp24::launch_mvue(static_cast<const uint16_t*>(M), U, rows, cols, static_cast<uint16_t*>(vals),
                                         meta, as_stream(stream)));
}

const char* sp24_status_str(int status) {
  switch (status) {
    case SP24_OK: return "ok";
    case SP24_ERR_NULL: return "null pointer";
    case SP24_ERR_SHAPE: return "bad shape (negative, or not a required multiple)";
    case SP24_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case SP24_ERR_LAUNCH: return "kernel launch failed";
    case SP24_ERR_UNSUPPORTED: return "unsupported";
    case SP24_ERR_TOO_LARGE: return "size exceeds index range";
    default: return "unknown status";
  }
}

int sp24_pattern_table(uint16_t* out) {
  if (out == nullptr) return SP24_ERR_NULL;
  for (int p = 0; p < sp24::kNumPatterns; ++p) out[p] = sp24::kTables.mask[p];
  return SP24_OK;
}

int sp24_abi_version(void) { return 8; }

}  // extern "C"
