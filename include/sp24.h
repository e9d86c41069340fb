/*
 * sp24.h - C ABI of the transposable 2:4 sparse FFN kernels for MI355X (gfx950).
 *
 * Method: "Accelerating Transformer Pre-training with 2:4 Sparsity" (Hu, Zhao,
 * Huang, Chen, Zhu; ICML 2024).  Citations below name the part of that paper's
 * pages that defines each operation:
 *   [Alg.1]    Algorithm 1, "transposable mask search" (reproducibility table,
 *              "Pseudocode" row): |W|, a stride-4 correlation with the mask
 *              patterns, argmax over patterns.
 *   [Abstract] the abstract: transposable 2:4 masks computed by convolution,
 *              2:4 sparse matrix multiplication for the FFN layers.
 *   [SW]       reproducibility table, "Software Dependencies" row: separate
 *              mask-search and pruning kernels, and 2:4 sparse MMs.
 *   [Decay]    the abstract's modified sparse-refined straight-through
 *              estimator, which applies the masked decay term on gradients,
 *              and the "Software Dependencies" row's masked-decay kernel.
 *              The pages give no formula; the library adds
 *              decay * (1 - M) * W to the straight-through weight gradient.
 *   [GEGLU]    the abstract's acceleration of gated activation functions and
 *              the "Software Dependencies" row's GEGLU kernel (no formula
 *              on the pages).
 *   [MVUE]     the "Software Dependencies" row's MVUE kernel (name only).
 *              The library's reading: the minimum-variance unbiased
 *              estimator that keeps 2 of 4 entries of a gradient.
 *   [Flip]     the abstract's "flip rate", a monitor of the stability of 2:4
 *              training.  The pages give no formula; the library counts the
 *              mask entries (of the R*C) whose kept/pruned state differs
 *              between two masks, and the rate is that count over R*C.
 *
 * Conventions shared by every entry point:
 *   - W is the fp16 weight [R, C], row-major, PyTorch Linear layout [out, in].
 *   - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *     caller.  The library allocates nothing, keeps no per-call state and never
 *     frees caller memory.  Buffers are contiguous and row-major, except the
 *     compressed 2:4 forms, which use the blocked order defined below.
 *   - Every device pointer must be 16-byte aligned (SP24_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue their kernels on that stream and return at once; nothing
 *     is synchronised.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation of that stream.  The stream and every buffer belong to
 *     the calling thread's current device (hipSetDevice), whose CU count
 *     picks the tiling.
 *   - Arguments are checked on the host before any HIP call, so every
 *     validation error is returned without touching the device.  A zero-sized
 *     problem (R, C or T equal to 0) is valid, launches nothing and may pass
 *     NULL for its buffers.
 *   - Calls are reentrant and thread-safe.
 *   - Inputs are expected to be finite.  +-Inf is handled deterministically
 *     (Inf scores tie and the first such pattern wins); NaN inputs give
 *     unspecified (but in-bounds) results.
 *
 * Pattern index: the 90 transposable 4x4 patterns (two kept entries in every
 * row and every column of the block) are numbered by the tuple (a, b, c, d) of
 * row-pair codes of rows 0..3, in lexicographic order, a slowest, with codes
 * 0:{0,1} 1:{0,2} 2:{0,3} 3:{1,2} 4:{1,3} 5:{2,3}.
 *
 * Compressed 2:4 storage (the pages leave the format open; this is the
 * library's fixed layout):
 *   row form     vals_row fp16 [R, C/2], meta_row uint16 [R, C/16].  Row i,
 *                group g (columns 4g..4g+3) keeps in-group positions i0 < i1:
 *                vals_row[i][2g] = W[i][4g+i0], vals_row[i][2g+1] = W[i][4g+i1]
 *                (bit copies), and the nibble (i0 | i1 << 2) sits at bits
 *                4*(g%4) .. 4*(g%4)+3 of meta_row[i][g/4].
 *   column form  vals_col fp16 [C, R/2], meta_col uint16 [C, R/16]: the same
 *                layout applied to the transpose of the pruned W (groups of 4
 *                along R).  It exists because the masks are transposable, so
 *                every column group keeps exactly two entries [Abstract].
 * The bracketed shapes above give the logical matrices; in memory each is
 * stored in BLOCKED ORDER (every vals and meta buffer of this library, in and
 * out), a permutation of the same number of elements:
 *   An n x m matrix (vals: m = C/2 halves per row, block width b = 32; meta:
 *   m = C/16 words per row, b = 4) is cut into bands of 64 rows (the last
 *   band has h = n - 64*(n/64) rows when n is not a multiple of 64).  Band k
 *   occupies elements [64*k*m, 64*k*m + h_k*m) and holds its column blocks
 *   of width b one after the other, each block row-major (h_k rows of its
 *   width; the last block of a row is m - b*(m/b) wide when b does not
 *   divide m).  So element (r, c) sits at
 *     64*k*m + b*(c/b)*h_k + (r - 64*k)*w + c%b,   k = r/64,
 *   with w = min(b, m - b*(c/b)).  One block holds the operands of 64
 *   columns of W (64 of the reduction) for 64 output rows, so a sparse
 *   product reads each of its stages as whole contiguous blocks.
 */
#ifndef SP24_H
#define SP24_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  SP24_OK = 0,
  SP24_ERR_NULL = 1,        /* a required pointer is NULL                        */
  SP24_ERR_SHAPE = 2,       /* negative size, or not a required multiple         */
  SP24_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned           */
  SP24_ERR_LAUNCH = 4,      /* the HIP runtime rejected a kernel launch          */
  SP24_ERR_UNSUPPORTED = 5, /* not available on this device / build              */
  SP24_ERR_TOO_LARGE = 6    /* a size exceeds the kernels' index range           */
};

/*
 * Transposable 2:4 mask search [Alg.1].
 *
 * For each 4x4 block (bi, bj) of |W| (rows 4bi..4bi+3, columns 4bj..4bj+3),
 * scores every pattern p as the fp32 sum of the 8 kept magnitudes added in
 * row-major order starting from +0, and writes the index of the first maximum
 * (strict >) to idx[bi * (C/4) + bj].  fp16 subnormals are kept exactly.
 *
 *   W    in   fp16 [R, C]
 *   R, C      R >= 0 and C >= 0, both multiples of 4 (a stride-4 window with
 *             no padding would drop a remainder; the call refuses it instead)
 *   idx  out  uint8 [R/4, C/4], values 0..89
 * Errors: NULL, SHAPE, ALIGN, TOO_LARGE (R*C >= 2^40), LAUNCH.
 */
int sp24_mask_search(const void* W, int64_t R, int64_t C, uint8_t* idx, void* stream);

/*
 * Prune W with the given masks and store both compressed forms [SW, Abstract].
 *
 *   W         in   fp16 [R, C]
 *   idx       in   uint8 [R/4, C/4] pattern indices (values >= 90 give
 *                  unspecified but in-bounds output)
 *   R, C           >= 0, both multiples of 16 (a meta word covers 4 groups)
 *   vals_row  out  fp16 [R, C/2]     meta_row  out  uint16 [R, C/16]
 *   vals_col  out  fp16 [C, R/2]     meta_col  out  uint16 [C, R/16]
 * Either (vals, meta) pair may be NULL to skip that form, but not both, and
 * not one pointer of a pair.
 * Errors: NULL, SHAPE, ALIGN, TOO_LARGE, LAUNCH.
 */
int sp24_compress(const void* W, const uint8_t* idx, int64_t R, int64_t C,
                  void* vals_row, uint16_t* meta_row,
                  void* vals_col, uint16_t* meta_col, void* stream);

/*
 * Mask search and compression in one pass over W [Alg.1, SW]: the same
 * results as sp24_mask_search followed by sp24_compress, with W read once.
 * idx may be NULL (not written).  Either (vals, meta) pair may be NULL, as in
 * sp24_compress.  R, C: >= 0, multiples of 16.
 * Errors: NULL, SHAPE, ALIGN, TOO_LARGE, LAUNCH.
 */
int sp24_search_compress(const void* W, int64_t R, int64_t C, uint8_t* idx,
                         void* vals_row, uint16_t* meta_row,
                         void* vals_col, uint16_t* meta_col, void* stream);

/*
 * One weight of a batched search + compression call.  W .. meta_col mean
 * what the arguments of sp24_search_compress mean; idx and either (vals,
 * meta) pair may be NULL, as there.
 *
 * Flip counting [Flip] (optional; both NULL to skip, both set to count):
 *   idx_prev  in   uint8 [R/4, C/4], the masks of the previous search (values
 *                  >= 90 are read as pattern 0).  It may be the same buffer as
 *                  idx, which is then updated in place (each block's previous
 *                  index is read before its new one is written), but it must
 *                  not overlap any other buffer of the call.
 *   flips     in/out  one uint64 in device memory, 8-byte aligned.  The call
 *                  ADDS the number of mask entries whose kept/pruned state
 *                  differs from idx_prev (an even number, at most R*C); the
 *                  caller clears it when it wants a fresh count, and several
 *                  jobs or calls may add into one counter.  The additions are
 *                  device atomics, so the total does not depend on order.
 */
typedef struct sp24_sc_job {
  const void* W;
  int64_t R;
  int64_t C;
  uint8_t* idx;
  void* vals_row;
  uint16_t* meta_row;
  void* vals_col;
  uint16_t* meta_col;
  const uint8_t* idx_prev;
  uint64_t* flips;
} sp24_sc_job;

#define SP24_MAX_BATCH 8

/*
 * sp24_search_compress for `count` weights (1..SP24_MAX_BATCH) in a single
 * kernel launch [Alg.1, SW]: an FFN layer re-searches both of its weights
 * every step, and one launch keeps the whole GPU streaming both.  `jobs` is a
 * HOST array, read during the call only.  Every job is validated first; on
 * any error nothing is launched and the first failing job's status is
 * returned.  Results are identical to separate sp24_search_compress calls.
 * Errors: NULL (jobs NULL, a job as in sp24_search_compress, or only one of
 * idx_prev and flips given), SHAPE (also count outside 1..SP24_MAX_BATCH),
 * ALIGN (flips needs 8 bytes, every other pointer 16), TOO_LARGE, LAUNCH.
 */
int sp24_search_compress_batch(const sp24_sc_job* jobs, int count, void* stream);

/*
 * Flip count between two mask-index arrays [Flip]: ADDS to *flips the number
 * of mask entries whose kept/pruned state differs between pattern idx_prev[i]
 * and pattern idx_new[i], summed over i in [0, nblocks).  Indices >= 90 are
 * read as pattern 0.  Dividing by 16*nblocks gives the flip rate.  The fused
 * form inside sp24_search_compress_batch saves this extra pass.
 *
 *   idx_prev, idx_new  in   uint8 [nblocks], 16-byte aligned
 *   nblocks                 >= 0, below 2^40
 *   flips     in/out  one uint64 in device memory, 8-byte aligned (as for
 *                     sp24_sc_job: the call adds, the caller clears)
 * Errors: NULL, SHAPE (negative nblocks), ALIGN, TOO_LARGE, LAUNCH.
 */
int sp24_flip_count(const uint8_t* idx_prev, const uint8_t* idx_new, int64_t nblocks,
                    uint64_t* flips, void* stream);

/*
 * Forward 2:4 sparse GEMM  Y = X * Ws^T  [Abstract, SW].
 *
 *   X         in   fp16 [T, C] activations
 *   vals_row, meta_row   in   row form of the pruned W [R, C]
 *   T, R, C        T >= 0; R, C >= 0 and multiples of 16
 *   Y         out  fp16 [T, R]; fp32 accumulation, rounded to nearest even
 * No bias, no activation.  Errors: NULL, SHAPE, ALIGN, TOO_LARGE, LAUNCH.
 */
int sp24_spmm_fwd(const void* X, const void* vals_row, const uint16_t* meta_row,
                  int64_t T, int64_t R, int64_t C, void* Y, void* stream);

/*
 * Forward 2:4 sparse GEMM of a gated FFN's first linear with GEGLU fused
 * into its epilogue [Abstract, SW, GEGLU]:
 *     U = X * Ws^T (fp16, as sp24_spmm_fwd), out = value * GELU(gate) of U
 * The rows of W (the output features of U) come in blocks of 32: rows
 * 32b .. 32b+15 are the value units 16b .. 16b+15 and rows 32b+16 .. 32b+31
 * their gate units, so U has sp24_geglu_fwd's layout with group 16.  `out`
 * is GEGLU of the fp16 products with the same fp32 GELU code as
 * sp24_geglu_fwd (the same inlined functions, no fp contraction), so it
 * equals sp24_geglu_fwd of U bit for bit.
 * Each value meets its gate in the same lane's accumulators, so U need not
 * be stored or read back.
 *
 *   X         in   fp16 [T, C]
 *   vals_row, meta_row   in   row form of the pruned W [R, C]
 *   T, R, C        as sp24_spmm_fwd, and R a multiple of 32
 *   U         out  fp16 [T, R], the products (for the backward), or NULL
 *   out       out  fp16 [T, R/2]
 * When C is not a multiple of 64, C is 4M or more, or an operand exceeds
 * 2 GiB, the library stores U and runs the GEGLU kernel on it; U must then be
 * given, else SP24_ERR_UNSUPPORTED.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, LAUNCH; TOO_LARGE as for
 * sp24_spmm_fwd, and when T*R/16 > 2^32 - 256 (the GEGLU kernel's launch).
 */
int sp24_spmm_fwd_geglu(const void* X, const void* vals_row, const uint16_t* meta_row,
                        int64_t T, int64_t R, int64_t C, void* U, void* out, void* stream);

/*
 * Input-gradient 2:4 sparse GEMM  dX = dY * Ws  [Abstract, SW].  Uses the
 * column form, which exists because the mask is transposable.
 *
 *   dY        in   fp16 [T, R]
 *   vals_col, meta_col   in   column form of the pruned W [R, C]
 *   T, R, C        as for sp24_spmm_fwd
 *   dX        out  fp16 [T, C]; fp32 accumulation, rounded to nearest even
 * Errors: NULL, SHAPE, ALIGN, TOO_LARGE, LAUNCH.
 */
int sp24_spmm_bwd_input(const void* dY, const void* vals_col, const uint16_t* meta_col,
                        int64_t T, int64_t R, int64_t C, void* dX, void* stream);

/*
 * Several independent 2:4 sparse GEMMs in one launch [Abstract, SW]: for
 * each entry g of gemms[0..count),
 *     out[T][N] = A[T][K] * S^T,
 * S the [N, K] matrix whose 2:4 row form (groups of 4 along K) is
 * (vals, meta).  The forward product of a layer is {A = X, (vals, meta) =
 * its row form, N = R, K = C}; its input gradient is {A = dY, (vals, meta) =
 * its column form, N = C, K = R}.  Each output equals the corresponding
 * sp24_spmm_fwd / sp24_spmm_bwd_input result bit for bit.
 * One persistent launch serves every product whose K is a multiple of 64
 * and at least 192 (and whose operands each stay below 2 GiB): its
 * workgroups take 256 x 256 output tiles from per-XCD queues, the
 * products with the longest K first, so the tiles of all products share
 * the GPU without a partly filled last round per product.  Other products
 * run as single launches before it.
 *
 *   gemms     in   host array of `count` descriptors (1..SP24_MAX_GROUP)
 *   workspace in   device memory of SP24_GROUP_WORKSPACE_BYTES bytes that
 *                  must be all zero before the first call (e.g. from
 *                  hipMemset); every call that completes leaves it all zero
 *                  again.  Calls that overlap in time must use different
 *                  workspaces.
 * The products must be independent: no output may overlap any input or
 * another output.  Per product: N, K multiples of 16, T >= 0, the buffers as
 * for sp24_spmm_fwd; an empty product (T or N zero) is skipped.
 * Errors: NULL, SHAPE (also count outside 1..SP24_MAX_GROUP), ALIGN,
 * TOO_LARGE, LAUNCH.
 */
typedef struct sp24_gemm {
  const void* A;           /* fp16 [T, K] */
  const void* vals;        /* fp16 [N, K/2] */
  const uint16_t* meta;    /* uint16 [N, K/16] */
  void* out;               /* fp16 [T, N] */
  int64_t T, N, K;
} sp24_gemm;

#define SP24_MAX_GROUP 8
#define SP24_GROUP_WORKSPACE_BYTES 64

int sp24_spmm_group(const sp24_gemm* gemms, int count, void* workspace, void* stream);

/*
 * sp24_spmm_group without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The queue counters live in the
 * library's own device array of SP24_GROUP_WORKSPACE_BYTES bytes, one copy
 * per GPU, held until the process ends: zero when the library is loaded,
 * and left zero by every call that completes.  Its device address is looked
 * up (hipGetSymbolAddress) on a device's first call.  The call allocates and
 * frees nothing.  Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (on different streams) race and must not be
 * made.  Same products, results (bit for bit) and limits as
 * sp24_spmm_group: up to SP24_MAX_GROUP products, SP24_ERR_SHAPE beyond.
 * Errors: as sp24_spmm_group; LAUNCH also when the array's address cannot be
 * had.
 */
int sp24_spmm_group_noalloc(const sp24_gemm* gemms, int count, void* stream);

/*
 * Weight gradient of a 2:4 FFN linear layer with the masked decay term
 * [Decay]:
 *     dW[r][c] = sum_t dY[t][r] * X[t][c]  +  decay * (1 - M[r][c]) * W[r][c]
 * The straight-through gradient reaches the dense weight W as the dense
 * product dY^T X (fp16 products, fp32 accumulation); M is the transposable
 * mask (1 where kept) given by idx.
 *
 *   dY        in   fp16 [T, R] output gradient of the layer
 *   X         in   fp16 [T, C] input of the layer
 *   W         in   fp16 [R, C] dense weight, or NULL (no decay term)
 *   idx       in   uint8 [R/4, C/4] pattern indices (values >= 90 read as 0),
 *                  NULL exactly when W is NULL
 *   decay          the decay factor (fp32)
 *   T, R, C        T >= 0; R, C >= 0, multiples of 16; T*R and T*C < 2^30
 *   dW        out  fp32 [R, C] (written, not accumulated).  T == 0 gives the
 *                  decay term alone (zeros without W).
 * Results are deterministic.  Every output element is reduced in a fixed
 * order by one workgroup, or, when the weight has too few tiles to fill the
 * GPU (a GPT-2-1.5B FFN weight), by two: each sums one half of the tokens in
 * a fixed order, and the second half's sum, stored in dW and announced by a
 * flag, is added to the first half's (fp32 addition of two terms does not
 * depend on their order).  The flags are library memory on each GPU (64
 * sets, taken in turn by the calls that split, each left clear); up to 64
 * such calls may overlap in time on one GPU.
 * Errors: NULL (also exactly one of W and idx given), SHAPE, ALIGN,
 * TOO_LARGE, LAUNCH (also when the flags' address cannot be had).
 */
int sp24_weight_grad(const void* dY, const void* X, const void* W, const uint8_t* idx, float decay,
                     int64_t T, int64_t R, int64_t C, float* dW, void* stream);

/*
 * GEGLU forward [GEGLU]: out[t][j] = value[t][j] * GELU(gate[t][j]), GELU the
 * exact x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), fp32 arithmetic, fp16
 * result rounded to nearest even.  Phi is evaluated within 7e-7 relative of
 * its exact value; gates of +-inf give what x * Phi(x) gives in IEEE
 * arithmetic (+inf, and NaN for -inf).
 *
 *   U      in   fp16 [T, 2h], the first linear's output.  Its columns come in
 *               blocks of `group` value columns followed by the `group`
 *               matching gate columns: value j is column
 *               2*group*(j/group) + j%group, its gate is `group` columns
 *               later.  group = h is the two-halves layout [value | gate].
 *   T, h, group  T >= 0; h >= 0 and group > 0, multiples of 8; h % group == 0
 *   out    out  fp16 [T, h]
 * Errors: NULL, SHAPE, ALIGN, LAUNCH; TOO_LARGE when T*2h >= 2^40 or when
 * T*h/8 > 2^32 - 256 (one work-item per 8 units, the most one launch takes).
 */
int sp24_geglu_fwd(const void* U, int64_t T, int64_t h, int64_t group, void* out, void* stream);

/*
 * GEGLU backward [GEGLU]: dU in U's layout, with
 *   d value = dout * GELU(gate),  d gate = dout * value * GELU'(gate),
 *   GELU'(x) = Phi(x) + x * phi(x).
 *   U      in   fp16 [T, 2h] as for sp24_geglu_fwd
 *   dout   in   fp16 [T, h]
 *   dU     out  fp16 [T, 2h] (may not overlap U or dout)
 * Errors: as sp24_geglu_fwd.
 */
int sp24_geglu_bwd(const void* U, const void* dout, int64_t T, int64_t h, int64_t group,
                   void* dU, void* stream);

/*
 * MVUE 2:4 estimate of a gradient [MVUE]: every group of 4 consecutive
 * entries a_0..a_3 of a row keeps exactly two, chosen at random so that the
 * estimate is unbiased with the least summed variance.
 *   - Keep probabilities: p_i = 2|a_i| / S with S = sum |a_i|, summed left to
 *     right.  If some p_k > 1, p_k = 1 and the others are |a_j| / (S - |a_k|).
 *   - Sampling: the cumulative sums C_0 = p_0, C_1 = C_0 + p_1,
 *     C_2 = C_1 + p_2 split [0, 2).  The picks are i = #{C_j <= u} and
 *     k = #{C_j <= u + 1}.  Rounding can put u in the last interval
 *     (i == 3, which exact arithmetic never does, as u < 1 <= C_2); u + 1 is
 *     then there too, and the picks are (i, k) = (2, 3).  Before the last
 *     interval, u + 1 always lies past u's: every p_j <= 1, and the fp32
 *     evaluation below keeps that order.
 *   - Kept values are a_i / p_i (0 where p_i == 0).  A group with fewer than
 *     two non-zero entries keeps its non-zero entry (if any) and the lowest
 *     other index, unchanged.
 * Evaluation, all fp32, in this order, without division: with D = S/2
 * (uncapped) or D = S - |a_k| (capped k, the first with 2|a_k| > S; the sum of
 * the other three left to right), masses w_j = |a_j| (w_k = D) and their
 * running sums W_0..W_2, the test C_j <= u is W_j <= u*D and C_j <= u + 1 is
 * W_j <= u*D + D.  A kept value is a_k for the capped entry and +-D (the sign
 * of a_j) for any other non-zero entry: a_j / p_j in exact arithmetic.
 * Values are rounded to nearest even in fp16, so results are reproducible bit
 * for bit.  An estimate beyond the fp16 range (|D| > 65504) becomes +-inf.
 *
 *   M      in   fp16 [rows, cols], the gradient (finite)
 *   U      in   fp32 [rows, cols/4], one uniform u in [0, 1) per group,
 *               supplied by the caller
 *   rows, cols   >= 0, cols a multiple of 16
 *   vals   out  fp16 [rows, cols/2]    meta  out  uint16 [rows, cols/16]
 *               The library's 2:4 row form in blocked order: the kept pair
 *               of group g in order, and its nibble i | k << 2.  The sparse
 *               GEMMs accept it as their sparse operand.
 * Errors: NULL, SHAPE, ALIGN, LAUNCH; TOO_LARGE when a dimension reaches
 * 2^31, rows*cols reaches 2^40, or ceil(rows/64) * ceil(cols/256) > 2^24 - 1
 * (one workgroup of 256 work-items per 64 x 256 panel; one launch takes at
 * most 2^32 - 256 work-items).
 */
int sp24_mvue(const void* M, const float* U, int64_t rows, int64_t cols, void* vals, uint16_t* meta,
              void* stream);

/* Host only: a static, human-readable name for a status code. */
const char* sp24_status_str(int status);

/*
 * Host only: writes the 90 patterns in index order to out[0..89] (host
 * memory).  Bit 4r+c of out[p] is set when pattern p keeps entry (r, c) of
 * the block.  Returns SP24_OK, or SP24_ERR_NULL for a NULL out.
 */
int sp24_pattern_table(uint16_t* out);

/* Host only: the library's ABI version (8 for this header). */
int sp24_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SP24_H */
