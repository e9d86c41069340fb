/*
 * Plain C client of the hot path on a GPU.  It includes only include/sp24.h
 * and the HIP runtime's C API, allocates with hipMalloc, and calls
 * sp24_search_compress, sp24_spmm_fwd and sp24_spmm_bwd_input on the null
 * stream, with no Python or torch in the process.
 *
 * Usage: hot_path DIR R C T
 *   reads  DIR/W.bin (fp16 [R][C]), DIR/X.bin (fp16 [T][C]), DIR/dY.bin (fp16 [T][R])
 *   writes DIR/idx.bin, vals_row.bin, meta_row.bin, vals_col.bin, meta_col.bin,
 *          DIR/Y.bin (fp16 [T][R]) and DIR/dX.bin (fp16 [T][C])
 * Prints "ok" and exits 0 on success; prints the failing step and exits 1
 * otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "sp24.h"

enum { N_BUF = 10 };
static void* dev_buf[N_BUF];
static int n_dev = 0;

static int fail(const char* what, const char* detail) {
  printf("FAILED %s: %s\n", what, detail);
  return 1;
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  if (bytes == 0) bytes = 16;
  if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
  dev_buf[n_dev++] = p;
  return p;
}

static int load(const char* dir, const char* name, void* dst, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return 0;
  void* host = malloc(bytes ? bytes : 1);
  const size_t got = fread(host, 1, bytes, f);
  fclose(f);
  const int ok = got == bytes && hipMemcpy(dst, host, bytes, hipMemcpyHostToDevice) == hipSuccess;
  free(host);
  return ok;
}

static int save(const char* dir, const char* name, const void* src, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  void* host = malloc(bytes ? bytes : 1);
  if (hipMemcpy(host, src, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 0;
  }
  FILE* f = fopen(path, "wb");
  const int ok = f && fwrite(host, 1, bytes, f) == bytes;
  if (f) fclose(f);
  free(host);
  return ok;
}

int main(int argc, char** argv) {
  int st, i, rc = 0;
  if (argc != 5) return fail("usage", "hot_path DIR R C T");
  const char* dir = argv[1];
  const int64_t R = atoll(argv[2]), C = atoll(argv[3]), T = atoll(argv[4]);
  if (R <= 0 || C <= 0 || T < 0) return fail("usage", "R, C > 0 and T >= 0");

  const size_t w_bytes = (size_t)(R * C * 2), idx_bytes = (size_t)((R / 4) * (C / 4));
  const size_t vr_bytes = (size_t)(R * (C / 2) * 2), mr_bytes = (size_t)(R * (C / 16) * 2);
  const size_t vc_bytes = (size_t)(C * (R / 2) * 2), mc_bytes = (size_t)(C * (R / 16) * 2);
  const size_t x_bytes = (size_t)(T * C * 2), y_bytes = (size_t)(T * R * 2);

  void* W = dev_alloc(w_bytes);
  uint8_t* idx = (uint8_t*)dev_alloc(idx_bytes);
  void* vals_row = dev_alloc(vr_bytes);
  uint16_t* meta_row = (uint16_t*)dev_alloc(mr_bytes);
  void* vals_col = dev_alloc(vc_bytes);
  uint16_t* meta_col = (uint16_t*)dev_alloc(mc_bytes);
  void* X = dev_alloc(x_bytes);
  void* dY = dev_alloc(y_bytes);
  void* Y = dev_alloc(y_bytes);
  void* dX = dev_alloc(x_bytes);
  if (n_dev != N_BUF) return fail("hipMalloc", "out of device memory");

  if (!load(dir, "W.bin", W, w_bytes) || !load(dir, "X.bin", X, x_bytes) || !load(dir, "dY.bin", dY, y_bytes)) {
    rc = fail("load", "an input file is missing or short");
    goto out;
  }
  st = sp24_search_compress(W, R, C, idx, vals_row, meta_row, vals_col, meta_col, NULL);
  if (st != SP24_OK) {
    rc = fail("sp24_search_compress", sp24_status_str(st));
    goto out;
  }
  st = sp24_spmm_fwd(X, vals_row, meta_row, T, R, C, Y, NULL);
  if (st != SP24_OK) {
    rc = fail("sp24_spmm_fwd", sp24_status_str(st));
    goto out;
  }
  st = sp24_spmm_bwd_input(dY, vals_col, meta_col, T, R, C, dX, NULL);
  if (st != SP24_OK) {
    rc = fail("sp24_spmm_bwd_input", sp24_status_str(st));
    goto out;
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    rc = fail("hipDeviceSynchronize", "a kernel failed");
    goto out;
  }
  if (!save(dir, "idx.bin", idx, idx_bytes) || !save(dir, "vals_row.bin", vals_row, vr_bytes) ||
      !save(dir, "meta_row.bin", meta_row, mr_bytes) || !save(dir, "vals_col.bin", vals_col, vc_bytes) ||
      !save(dir, "meta_col.bin", meta_col, mc_bytes) || !save(dir, "Y.bin", Y, y_bytes) ||
      !save(dir, "dX.bin", dX, x_bytes)) {
    rc = fail("save", "could not write an output file");
    goto out;
  }
  printf("ok\n");
out:
  for (i = 0; i < n_dev; ++i) hipFree(dev_buf[i]);
  return rc;
}
