// Weight gradient of a 2:4 FFN linear layer with the masked decay term, for
// gfx950 matrix cores.
//
//   dW[r][c] = sum_t dY[t][r] * X[t][c]  +  decay * (1 - M[r][c]) * W[r][c]
//
// "Accelerating Transformer Pre-training with 2:4 Sparsity": the abstract
// modifies the sparse-refined straight-through estimator by applying the
// masked decay term on gradients, and the reproducibility table's "Software
// Dependencies" row lists a masked-decay kernel.  The straight-through
// gradient of the dense weight is the dense product dY^T X; the decay term
// (M the transposable mask, 1 where kept) is added to it in the epilogue, so
// the gradient is written once.  Output fp32 [R][C].
//
// The reduction runs over tokens, the slow axis of both operands in HBM
// (dY [T][R], X [T][C]), so neither operand is contiguous along K.  Rows of
// both are copied as they are into LDS by direct global->LDS loads, and the
// gfx950 transpose read ds_read_b64_tr_b16 turns them into MFMA fragments:
// within each 16-lane group it hands lane i element i of four 16-half rows,
// row j being the 8-byte chunks addressed by lanes 4j .. 4j+3.  Lane i of a
// group therefore addresses LDS row k0 + i/4 at column m0 + 4*(i%4), and
// receives A[m0 + i][k0 .. k0+3].
//
// v_mfma_f32_32x32x16_f16 operands (lane l, g = l / 32):
//   A: row l % 32 (the weight row r), k in [8g, 8g + 8)   (two transpose reads)
//   B: column l % 32 (the weight column c), k in [8g, 8g + 8)
//   D: column l % 32, rows 8*(i/4) + 4g + i%4 for accumulator i
// Each group of four accumulators is four consecutive rows of one column
// inside one 4x4 mask block, which the decay epilogue uses.
//
// Tiling: a workgroup computes BM rows x BN columns of dW with four waves
// (one per SIMD) of WM x WN, K (tokens) in stages of 32 through a 3-stage
// LDS ring filled two stages ahead.  Rows of dY/X past T read as zero (buffer
// bounds); columns past R or C feed only outputs that are not stored.
//
// Token split: when a weight has too few tiles to fill the GPU (256 x 320
// tiles of a GPT-2-1.5B FFN weight: 125 on 256 CUs), each tile runs as two
// workgroups, one per half of the tokens.  The second half's workgroup (the
// producer) stores its partial product into dW and raises the tile's flag;
// the first half's (the consumer) waits for the flag, adds the stored partial
// to its own and adds the decay term.  Two fp32 partials sum to the same
// value in either order, so the result does not depend on timing.  Producers
// never wait; they run on XCDs 0-3 and the consumers on XCDs 4-7 (workgroup
// id modulo 8), so a waiting consumer never holds a CU its producer needs,
// and the wait always ends.  Were all workgroups to reach a single queue, a
// producer's id is still the lower (by 4), and workgroups start in id order.
// An XCD then computes twice the tiles over half the tokens, whose operand
// strips are fewer bytes than those of half the tiles over all of them.  The
// consumer's wait is bounded all the same (about 0.1 s).
#include <hip/hip_runtime.h>
#include <atomic>
#include <cstdint>

#include "sp24_device.hpp"
#include "sp24_internal.hpp"
#include "sp24_patterns.hpp"

namespace sp24 {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr int kBK = 32;   // tokens per stage

struct MaskTable {
  uint16_t mask[kNumPatterns + 2];   // kept entries of each pattern, bit 4r+c
};
constexpr MaskTable build_mask_table() {
  MaskTable t{};
  for (int p = 0; p < kNumPatterns; ++p) t.mask[p] = kTables.mask[p];
  return t;
}
__constant__ MaskTable g_masks = build_mask_table();

template <int BM, int BN, int WM, int WN>
struct DwCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = kBK * BM * 2, B_BYTES = kBK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024, B_LOADS = B_BYTES / 1024;   // 1 KiB direct loads
  static constexpr int NLOADS = A_LOADS + B_LOADS;
  static constexpr int LOADS_HI = (NLOADS + WAVES - 1) / WAVES;   // per wave (the first NLOADS % WAVES waves)
  static constexpr int LOADS_LO = NLOADS / WAVES;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % WM == 0 && BN % WN == 0, "tile shape");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "rows must split into whole direct loads");
  static_assert(LOADS_HI <= 15, "vmcnt immediate");
  static constexpr size_t SMEM = 3 * (size_t)STAGE + sizeof(MaskTable);
};

// LDS row layout of a stage: a row of `slots` 16-byte chunks (the chunk of
// columns 8q .. 8q+7 is q) stores chunk q at slot (q + rot(row & 3)) % slots.
// The LDS serves 32 lanes of a read per cycle from 64 four-byte banks, and
// the 32 lanes of a transpose read fetch two 32-byte windows (q even, and
// q + 2) in each of four consecutive rows.  The rotation makes the window
// offsets of rows j = 0..3 congruent to 64*j bytes modulo 256, so the eight
// windows cover the 64 banks once (checked for the row sizes used below).
constexpr int rot_slots(int row_bytes, int j) { return ((4 - row_bytes / 16) * j % 16 + 16) % 16; }
constexpr bool windows_disjoint(int row_bytes) {
  bool used[16] = {};
  for (int j = 0; j < 4; ++j)
    for (int p = 0; p < 2; ++p) {
      const int slot = (j * row_bytes / 16 + rot_slots(row_bytes, j) + 2 * p) % 16;
      if (used[slot] || used[(slot + 1) % 16]) return false;
      used[slot] = used[(slot + 1) % 16] = true;
    }
  return true;
}
static_assert(windows_disjoint(512) && windows_disjoint(320) && windows_disjoint(256) && windows_disjoint(640),
              "bank-disjoint windows");

// vmcnt wait (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Token-split roles
enum : int { kWhole = 0, kConsumer = 1, kProducer = 2 };

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN), 1) void weight_grad_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    const uint8_t* __restrict__ idx, float decay, int64_t T, int64_t R, int64_t C, float* __restrict__ dW,
    int tiles_m, int tiles_n, int split, unsigned int* __restrict__ flags) {
  using Cfg = DwCfg<BM, BN, WM, WN>;
  __shared__ __align__(1024) unsigned char smem[Cfg::SMEM];
  MaskTable* masks = reinterpret_cast<MaskTable*>(smem + 3 * Cfg::STAGE);

  // Workgroups are dealt round-robin to the 8 XCDs; each XCD takes a
  // contiguous run of tiles.  Whole tiles: runs of ceil(tiles/8) in groups of
  // 8 row tiles, column tiles within a group.  Split: XCD x < 4 runs the
  // producers of run x (ceil(tiles/4) tiles), XCD x + 4 their consumers, both
  // over half the tokens, with the tiles taken across the grid's shorter side
  // first, so that each XCD's L2 fetches the operand strips of a compact block.
  const int ntiles = tiles_m * tiles_n;
  const int xcd = (int)(blockIdx.x % 8), in_xcd = (int)(blockIdx.x / 8);
  int role = kWhole, lin, tm, tn;
  if (split) {
    const int per_run = (ntiles + 3) / 4;
    role = xcd < 4 ? kProducer : kConsumer;
    lin = (xcd % 4) * per_run + in_xcd;
    if (in_xcd >= per_run || lin >= ntiles) return;
    if (tiles_n <= tiles_m) {
      tm = lin / tiles_n;
      tn = lin % tiles_n;
    } else {
      tn = lin / tiles_m;
      tm = lin % tiles_m;
    }
  } else {
    constexpr int kGroupM = 8;
    const int per_xcd = (ntiles + 7) / 8;
    lin = xcd * per_xcd + in_xcd;
    if (in_xcd >= per_xcd || lin >= ntiles) return;
    const int group = lin / (kGroupM * tiles_n);
    const int gm0 = group * kGroupM;
    const int gsize = min(kGroupM, tiles_m - gm0);
    const int in_group = lin - group * kGroupM * tiles_n;
    tn = in_group / gsize;
    tm = gm0 + in_group % gsize;
  }
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WAVES_M, wn = wave / Cfg::WAVES_M;
  // stages of 32 tokens: the consumer takes the first half, the producer the rest
  const int nk_all = (int)((T + kBK - 1) / kBK);
  const int k_lo = role == kProducer ? nk_all / 2 : 0;
  const int nk = role == kWhole ? nk_all : role == kConsumer ? nk_all / 2 : nk_all - nk_all / 2;
  const int64_t t0 = (int64_t)k_lo * kBK;

  if (tid < (int)(sizeof(MaskTable) / 4))
    reinterpret_cast<uint32_t*>(masks)[tid] = reinterpret_cast<const uint32_t*>(&g_masks)[tid];

  // buffer descriptors from this tile's first column (at token t0) to the
  // matrix end; bytes past it (token rows beyond T) load as zero
  const i32x4 ra = make_rsrc(dY + t0 * R + m0, (uint32_t)(((T - t0) * R - m0) * 2));
  const i32x4 rb = make_rsrc(X + t0 * C + n0, (uint32_t)(((T - t0) * C - n0) * 2));

  // This wave's direct loads: loads w, w + WAVES, ... of a stage.  Load j
  // fills LDS slots 64j .. 64j+63 (16 bytes each) of the stage, A rows first;
  // each lane fetches the chunk that the rotation puts in its slot.
  const int nl = wave < Cfg::NLOADS % Cfg::WAVES ? Cfg::LOADS_HI : Cfg::LOADS_LO;
  int goff[Cfg::LOADS_HI];
#pragma unroll
  for (int u = 0; u < Cfg::LOADS_HI; ++u) {
    const int j = wave + u * Cfg::WAVES;
    goff[u] = 0;
    if (j < Cfg::A_LOADS) {
      constexpr int n = BM / 8;
      const int s = 64 * j + lane, row = s / n, slot = s % n;
      goff[u] = row * (int)R * 2 + ((slot + n - rot_slots(2 * BM, row & 3)) % n) * 16;
    } else if (j < Cfg::NLOADS) {
      constexpr int n = BN / 8;
      const int s = 64 * (j - Cfg::A_LOADS) + lane, row = s / n, slot = s % n;
      goff[u] = row * (int)C * 2 + ((slot + n - rot_slots(2 * BN, row & 3)) % n) * 16;
    }
  }
  auto issue_one = [&](int u, int kt, int slot_ring) {
    const int j = wave + u * Cfg::WAVES;
    const uint32_t dst = lds_addr(smem) + slot_ring * Cfg::STAGE + 1024 * j;
    if (j < Cfg::A_LOADS)
      dma_b128(ra, dst, goff[u] + kt * kBK * (int)R * 2);
    else
      dma_b128(rb, dst, goff[u] + kt * kBK * (int)C * 2);
  };
  auto issue = [&](int kt, int slot_ring) {
#pragma unroll
    for (int u = 0; u < Cfg::LOADS_HI; ++u)
      if (u < nl) issue_one(u, kt, slot_ring);
  };
  // allow `stages` stages of this wave's loads to stay in flight
  auto wait_loads = [&](int stages) {
    if (stages == 0) {
      wait_vm<0>();
    } else if (nl == Cfg::LOADS_HI) {
      if (stages >= 2) wait_vm<2 * Cfg::LOADS_HI>(); else wait_vm<Cfg::LOADS_HI>();
    } else {
      if (stages >= 2) wait_vm<2 * Cfg::LOADS_LO>(); else wait_vm<Cfg::LOADS_LO>();
    }
  };

  // transpose-read offsets of this lane inside a stage, per 32-row block:
  // lane i of 16-lane group G addresses row 8*(G/2) + i/4 (+ 16 per k16 step,
  // + 4 for the second half) at column 32*block + 16*(G%2) + 4*(i%4)
  const int G = lane >> 4, i16 = lane & 15, j4 = i16 >> 2, c4 = i16 & 3;
  const int krow = 8 * (G >> 1) + j4;
  int a_off[Cfg::TM], b_off[Cfg::TN];
#pragma unroll
  for (int mt = 0; mt < Cfg::TM; ++mt) {
    constexpr int n = BM / 8;
    const int q = (wm * WM + mt * 32 + 16 * (G & 1)) / 8 + (c4 >> 1);
    a_off[mt] = krow * (2 * BM) + ((q + rot_slots(2 * BM, j4)) % n) * 16 + (c4 & 1) * 8;
  }
#pragma unroll
  for (int nt = 0; nt < Cfg::TN; ++nt) {
    constexpr int n = BN / 8;
    const int q = (wn * WN + nt * 32 + 16 * (G & 1)) / 8 + (c4 >> 1);
    b_off[nt] = Cfg::A_BYTES + krow * (2 * BN) + ((q + rot_slots(2 * BN, j4)) % n) * 16 + (c4 & 1) * 8;
  }

  // With five row or column blocks (waves of 128 x 160 or 160 x 128) the 20
  // accumulator tiles exceed the 256 accumulation registers: the fifth block
  // runs as an asm MFMA with its accumulators in ordinary VGPRs (the compiler
  // gives every MFMA builtin of a function the same register form).
  constexpr bool kAsmN = Cfg::TN == 5, kAsmM = Cfg::TM == 5;
  static_assert(Cfg::TM * Cfg::TN <= 16 || kAsmN || kAsmM, "accumulators beyond the AGPRs");
  f16v acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  struct Frags {
    h8 a[Cfg::TM];
    h8 b[Cfg::TN];
  };
  auto tr_read = [&](int byte) -> h4 {
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)((lds_u8*)smem + byte)));
  };
  // fragments of k16 step ks (0 or 1) of the stage in ring slot `sl`
  auto load_frags = [&](int sl, int ks, Frags& f) {
    const int base = sl * Cfg::STAGE;
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt) {
      const int o = base + a_off[mt] + ks * 16 * (2 * BM);
      const h4 lo = tr_read(o), hi = tr_read(o + 4 * (2 * BM));
      f.a[mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int nt = 0; nt < Cfg::TN; ++nt) {
      const int o = base + b_off[nt] + ks * 16 * (2 * BN);
      const h4 lo = tr_read(o), hi = tr_read(o + 4 * (2 * BN));
      f.b[nt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // the MFMAs of one k16 step; when kt_load >= 0 this wave's direct loads of
  // stage kt_load go out one per MFMA so the texture path drains steadily
  auto mfmas = [&](const Frags& f, int kt_load, int slot_ring) {
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        if ((kAsmN && nt == 4) || (kAsmM && mt == 4)) {
          // s_nop 1: wait states after a VALU write of the operands
          asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                       : "+v"(acc[mt][nt])
                       : "v"(f.a[mt]), "v"(f.b[nt]));
        } else {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[mt], f.b[nt], acc[mt][nt], 0, 0, 0);
        }
        const int u = mt * Cfg::TN + nt;
        if (u < Cfg::LOADS_HI && kt_load >= 0 && u < nl) issue_one(u, kt_load, slot_ring);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int u = Cfg::TM * Cfg::TN; u < Cfg::LOADS_HI; ++u)
      if (kt_load >= 0 && u < nl) issue_one(u, kt_load, slot_ring);
  };

  if (nk > 0) {
    // Pipeline: stage s goes to ring slot s % 3, three stages ahead.  In
    // stage kt the second k16 step's fragments are read during the first
    // step's MFMAs; mid-stage the wave waits for stage kt+1, all waves meet
    // (nobody reads slot kt % 3 afterwards), stage kt+3 is issued into it,
    // and stage kt+1's first fragments are read during the second step.
    for (int s = 0; s < 3; ++s)
      if (s < nk) issue(s, s);
    wait_loads(min(nk, 3) - 1);
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
    load_frags(0, 0, f0);
    auto stage = [&](int kt, int cur, int nxt) {
      load_frags(cur, 1, f1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f0, -1, 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_loads(kt + 2 < nk ? 1 : 0);
      // lgkmcnt(0): this wave's reads of slot kt % 3 are done before the
      // barrier lets stage kt+3 overwrite it
      __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < nk) load_frags(nxt, 0, f0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f1, kt + 3 < nk ? kt + 3 : -1, cur);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < nk; kt += 3) {
      stage(kt, 0, 1);
      if (kt + 1 < nk) stage(kt + 1, 1, 2);
      if (kt + 2 < nk) stage(kt + 2, 2, 0);
    }
  }
  __syncthreads();   // the mask table is visible (and the ring idle)
  // the asm MFMAs' results are read by VALU below: 18 or more wait states
  // after the last one
  if constexpr (kAsmN || kAsmM) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // Epilogue: each group of four accumulators is rows r4 .. r4+3 (one mask
  // block row) of column c; add the decay term to the pruned entries.
  const int l32 = lane & 31, g = lane >> 5;
  const bool with_decay = W != nullptr;
  unsigned int* const flag = split ? flags + lin : nullptr;
  if (role == kProducer) {
    // the raw partial of the second half of the tokens
#pragma unroll
    for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < Cfg::TN; ++nt) {
        const int64_t c = n0 + wn * WN + nt * 32 + l32;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int64_t r4 = m0 + wm * WM + mt * 32 + 8 * i4 + 4 * g;
          if (r4 >= R || c >= C) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) dW[(r4 + e) * C + c] = acc[mt][nt][4 * i4 + e];
        }
      }
    // every wave's stores are done, then they are made visible device-wide
    // before the flag goes up
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    __syncthreads();
    if (tid == 0) {
      __atomic_thread_fence(__ATOMIC_RELEASE);
      // the L2 write-back the fence issues has completed before the flag is stored
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (role == kConsumer) {
    if (tid == 0) {
      // bounded: 25000 sleeps of about 8000 clocks
      for (int spin = 0; spin < 25000; ++spin) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
        __builtin_amdgcn_s_sleep(127);
      }
      __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next launch
    }
    __syncthreads();
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
  }
  // The epilogue goes through the tile a 32-row block and two of its column
  // blocks at a time: every load of such a group (the producer's partial, the
  // block indices and W for the decay term) is issued before its first store,
  // so they are in flight together.  Loaded one element group at a time, the
  // consumer's epilogue took 170 us of a 480 us launch (its partial and W come
  // from memory after the acquire).  Addresses are clamped into the matrix;
  // values of elements outside it are loaded and never used.
  constexpr int kHalf = 2;   // column blocks per group
#pragma unroll
  for (int mt = 0; mt < Cfg::TM; ++mt)
#pragma unroll
    for (int part = 0; part < (Cfg::TN + kHalf - 1) / kHalf; ++part) {
      float prev[kHalf][16];
      uint32_t pat[kHalf][4];
      uint16_t wv[kHalf][16];
#pragma unroll
      for (int h = 0; h < kHalf; ++h) {
        const int nt = part * kHalf + h;
        if (nt >= Cfg::TN) continue;
        const int64_t c = min<int64_t>(n0 + wn * WN + nt * 32 + l32, C - 1);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int64_t r4 = min<int64_t>(m0 + wm * WM + mt * 32 + 8 * i4 + 4 * g, R - 4);
          if (role == kConsumer) {
#pragma unroll
            for (int e = 0; e < 4; ++e) prev[h][4 * i4 + e] = dW[(r4 + e) * C + c];   // the producer's partial
          }
          if (with_decay) {
            pat[h][i4] = idx[(r4 / 4) * (C / 4) + c / 4];
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[h][4 * i4 + e] = W[(r4 + e) * C + c];
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kHalf; ++h) {
        const int nt = part * kHalf + h;
        if (nt >= Cfg::TN) continue;
        const int64_t c = n0 + wn * WN + nt * 32 + l32;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int64_t r4 = m0 + wm * WM + mt * 32 + 8 * i4 + 4 * g;
          if (r4 >= R || c >= C) continue;
          float v[4] = {acc[mt][nt][4 * i4], acc[mt][nt][4 * i4 + 1], acc[mt][nt][4 * i4 + 2],
                        acc[mt][nt][4 * i4 + 3]};
          if (role == kConsumer) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += prev[h][4 * i4 + e];
          }
          if (with_decay) {
            uint32_t p = pat[h][i4];
            p = p < (uint32_t)kNumPatterns ? p : 0u;
            const uint32_t kept = (uint32_t)masks->mask[p] >> (c & 3);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (!((kept >> (4 * e)) & 1u)) v[e] = v[e] + decay * (float)__builtin_bit_cast(_Float16, wv[h][4 * i4 + e]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) dW[(r4 + e) * C + c] = v[e];
        }
      }
    }
}

struct DwShape {
  int bm, bn;
};

template <int BM, int BN, int WM, int WN>
hipError_t launch_dw(const uint16_t* dY, const uint16_t* X, const uint16_t* W, const uint8_t* idx, float decay,
                     int64_t T, int64_t R, int64_t C, float* dW, hipStream_t s, unsigned int* flags = nullptr) {
  using Cfg = DwCfg<BM, BN, WM, WN>;
  const int tiles_m = (int)((R + BM - 1) / BM), tiles_n = (int)((C + BN - 1) / BN);
  const int split = flags != nullptr ? 1 : 0;
  const int grid = 8 * (split ? (tiles_m * tiles_n + 3) / 4 : (tiles_m * tiles_n + 7) / 8);
  hipLaunchKernelGGL((weight_grad_kernel<BM, BN, WM, WN>), dim3(grid), dim3(Cfg::THREADS), 0, s, dY, X, W, idx, decay,
                     T, R, C, dW, tiles_m, tiles_n, split, flags);
  return hipGetLastError();
}

// Tile flags of the token split: 64 sets of kDwFlagTiles words in the library,
// one copy per GPU (zero when the library is loaded; each consumer clears its
// tile's flag).  Launches take the sets in turn, so launches that run at the
// same time on one GPU (from different streams) use different sets unless 64
// of them overlap.  The device address comes from hipGetSymbolAddress, looked
// up once per device with that device current.
constexpr int kDwFlagSets = 64, kDwFlagTiles = 256;
__device__ __align__(256) unsigned int dw_flags[kDwFlagSets * kDwFlagTiles];

hipError_t dw_flag_set(unsigned int** out) {
  static std::atomic<unsigned int*> ptrs[64];
  static std::atomic<unsigned int> next{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned int* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(dw_flags));
    if (e != hipSuccess) return e;
    ptrs[dev].store(p, std::memory_order_release);
  }
  *out = p + (size_t)(next.fetch_add(1, std::memory_order_relaxed) % kDwFlagSets) * kDwFlagTiles;
  return hipSuccess;
}

}  // namespace

hipError_t launch_weight_grad(const uint16_t* dY, const uint16_t* X, const uint16_t* W, const uint8_t* idx,
                              float decay, int64_t T, int64_t R, int64_t C, float* dW, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  // Tile shape: each candidate's time is modelled as (rounds of one tile per
  // CU) x (tile area / relative speed of the shape); the cheapest wins.  The
  // 256 x 320 and 320 x 256 tiles (waves of 128 x 160 or 160 x 128, the fewest
  // LDS bytes per MFMA) may split the tokens in two when twice their tiles
  // still fit on the CUs: a GPT-2-1.5B FFN weight (6400 x 1600 or 1600 x 6400)
  // is 125 such tiles, 250 workgroups on 256 CUs.
  struct Cand {
    int bm, bn;
    double speed;
    bool splittable;
  };
  const Cand cands[] = {{256, 256, 1.0, false}, {256, 320, 0.97, true}, {320, 256, 0.97, true},
                        {256, 160, 0.9, false}, {160, 256, 0.9, false}, {128, 128, 0.75, false}};
  constexpr int kCands = sizeof(cands) / sizeof(cands[0]);
  const int64_t cus = device_cu_count();
  const int64_t stages = (T + kBK - 1) / kBK;
  int best = 0;
  bool best_split = false;
  double best_t = 0.0;
  for (int k = 0; k < kCands; ++k) {
    const int64_t tiles = ((R + cands[k].bm - 1) / cands[k].bm) * ((C + cands[k].bn - 1) / cands[k].bn);
    const double area = (double)cands[k].bm * cands[k].bn / cands[k].speed;
    double t = (double)((tiles + cus - 1) / cus) * area;
    bool split = false;
    // split only whole tiles that fill at least three quarters of the CUs
    // with their halves: a 1600 x 3200 weight (70 ragged 256 x 320 tiles, 140
    // workgroups) took 310 us split against 274 us as 325 128 x 128 tiles
    const bool whole = R % cands[k].bm == 0 && C % cands[k].bn == 0;
    if (cands[k].splittable && whole && 2 * tiles <= cus && 8 * tiles >= 3 * cus && tiles <= kDwFlagTiles &&
        stages >= 2 && area / 2 < t) {
      t = area / 2;
      split = true;
    }
    if (k == 0 || t < best_t) {
      best = k;
      best_t = t;
      best_split = split;
    }
  }
  unsigned int* flags = nullptr;
  if (best_split) {
    const hipError_t e = dw_flag_set(&flags);
    if (e != hipSuccess) return e;
  }
  switch (best) {
    case 0: return launch_dw<256, 256, 128, 128>(dY, X, W, idx, decay, T, R, C, dW, s);
    case 1: return launch_dw<256, 320, 128, 160>(dY, X, W, idx, decay, T, R, C, dW, s, flags);
    case 2: return launch_dw<320, 256, 160, 128>(dY, X, W, idx, decay, T, R, C, dW, s, flags);
    case 3: return launch_dw<256, 160, 64, 160>(dY, X, W, idx, decay, T, R, C, dW, s);
    case 4: return launch_dw<160, 256, 160, 64>(dY, X, W, idx, decay, T, R, C, dW, s);
    default: return launch_dw<128, 128, 64, 64>(dY, X, W, idx, decay, T, R, C, dW, s);
  }
}

}  // namespace sp24
