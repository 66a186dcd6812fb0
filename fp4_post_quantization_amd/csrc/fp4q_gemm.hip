// W4A4 MXFP4 matrix product on gfx950's scaled FP4 matrix cores.
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (2. Metodologia; 3. QuTLASS): both operands of the product
// are FP4 with per-block scales.  On gfx950 the matrix core takes MXFP4
// directly: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32 x 64 block of
// A by a 64 x 32 block of B^T with E8M0 scales per 32 elements of K.  Lane l
// supplies row l % 32 and the 32 consecutive K elements starting at
// 32 * (l / 32): 16 bytes of codes in the storage order of a quantized row,
// plus that block's scale byte.  A row's stored bytes are therefore the
// matrix core's operand with no reordering.  The accumulator layout
// (register v of lane l holds row 8 (v / 4) + 4 (l / 32) + v % 4, column
// l % 32) and the operand layout were checked on the device.
//
// Two kernels:
//  * mx_gemm_ring_kernel (K a multiple of 128, the main path): 8 waves
//    compute a 256 x 256 tile, each wave 128 x 64 (4 x 2 accumulator
//    blocks, two waves per SIMD); smaller problems use 128 x 128 or 64 x 64
//    tiles.  K advances in stages of 128 or 64 bytes per row (256 or 128
//    MXFP4 elements; 64 or 32 bf16 values).  Stages travel from global
//    memory straight into an LDS ring (direct global-to-LDS loads), so the
//    next stages are in flight while one is consumed; 128-byte stages make
//    every load cover whole 128-byte lines.  Each wave reads a k step's operands while the previous k
//    step's MFMAs run.  The output tile leaves through LDS as 16-byte row
//    stores.
//  * mx_gemm_kernel (any K that is a multiple of 32): register-staged
//    double buffer, padded LDS rows, K tail zero-filled.
// Workgroups are renumbered so that each XCD (dispatched round-robin) gets
// a contiguous range of tiles, taken in groups of tile rows, and tiles that
// share A or B panels share an L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "fp4q_device.h"
#include "fp4q_gemm.h"

namespace fp4q_gemm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kKc = 128;     // K elements per stage
constexpr int kLdsRow = 80;  // bytes per staged row (64 + 16 padding)
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;  // tile rows per group in the tile order

// f(std::integral_constant<int, I>) for I = 0, 1, ..., N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void unroll(std::integer_sequence<int, I...>, F &&f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// float32 -> bfloat16, round to nearest even, two values per instruction (v_cvt_pk_bf16_f32: lo in
// the low half).  On every float32 pattern, in both halves, it gives what the integer rounding
// (b + 0x7FFF + lsb) >> 16 gives, and a NaN gives (b >> 16) | 0x40 (checked on the device over all
// 2^32 patterns).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((fp4q::f32x2{lo, hi}), bf16x2v));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.0f); }

__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

// Tile (tm, tn) of workgroup `id`: XCD-contiguous renumbering, then groups
// of kGroupRows tile rows walked column by column.
__device__ __forceinline__ void tile_of(int id, int total, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  const int lin = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int in_group = kGroupRows * tiles_n;
  const int group = lin / in_group;
  const int first = group * kGroupRows;
  const int gsize = min(tiles_m - first, kGroupRows);
  const int r = lin - group * in_group;
  tm = first + r % gsize;
  tn = r / gsize;
}

template <int TM, int TN, bool DWORD_SCALES, typename OutT>
__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(const uint8_t *__restrict__ A,
                                                           const uint8_t *__restrict__ As,
                                                           const uint8_t *__restrict__ B,
                                                           const uint8_t *__restrict__ Bs, int M, int N, int K,
                                                           float alpha, OutT *__restrict__ C, int64_t ldc) {
  constexpr int BM = 2 * TM * 32, BN = 2 * TN * 32;
  constexpr int PA = BM * 4 / kThreads, PB = BN * 4 / kThreads;  // 16-byte pieces per thread
  static_assert(PA >= 1 && PB >= 1, "tile too small for the staging layout");
  __shared__ __attribute__((aligned(16))) uint8_t lA[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lB[2][BN * kLdsRow];
  __shared__ uint32_t sA[2][BM], sB[2][BN];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2;        // code bytes per row
  const int ksc = K / 32;          // scale bytes per row
  const int nst = (K + kKc - 1) / kKc;

  i32x4 ra[PA], rb[PB];
  uint32_t rsa = 0x7F7F7F7Fu, rsb = 0x7F7F7F7Fu;

  auto load_scales = [&](const uint8_t *S, int rows, int r, int st) -> uint32_t {
    if (r >= rows) return 0x7F7F7F7Fu;
    const uint8_t *p = S + (int64_t)r * ksc + 4 * st;
    if constexpr (DWORD_SCALES) {
      return *reinterpret_cast<const uint32_t *>(p);
    } else {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) v |= (uint32_t)((4 * st + j < ksc) ? p[j] : 0x7F) << (8 * j);
      return v;
    }
  };
  auto gload = [&](int st) {
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      const int e = tid + kThreads * j, r = e >> 2, pc = e & 3;
      const bool ok = (m0 + r < M) && (st * kKc + 32 * pc < K);
      ra[j] = ok ? *reinterpret_cast<const i32x4 *>(A + (int64_t)(m0 + r) * kb + st * 64 + 16 * pc)
                 : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int e = tid + kThreads * j, r = e >> 2, pc = e & 3;
      const bool ok = (n0 + r < N) && (st * kKc + 32 * pc < K);
      rb[j] = ok ? *reinterpret_cast<const i32x4 *>(B + (int64_t)(n0 + r) * kb + st * 64 + 16 * pc)
                 : i32x4{0, 0, 0, 0};
    }
    if (tid < BM) rsa = load_scales(As, M, m0 + tid, st);
    if (tid < BN) rsb = load_scales(Bs, N, n0 + tid, st);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      const int e = tid + kThreads * j, r = e >> 2, pc = e & 3;
      *reinterpret_cast<i32x4 *>(&lA[buf][r * kLdsRow + 16 * pc]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int e = tid + kThreads * j, r = e >> 2, pc = e & 3;
      *reinterpret_cast<i32x4 *>(&lB[buf][r * kLdsRow + 16 * pc]) = rb[j];
    }
    if (tid < BM) sA[buf][tid] = rsa;
    if (tid < BN) sB[buf][tid] = rsb;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{0};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 a[TM], b[TN];
      int sa[TM], sb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + l32;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(&lA[buf][r * kLdsRow + 32 * ks + 16 * h]);
        a[i] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        sa[i] = (int)((sA[buf][r] >> (8 * (2 * ks + h))) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + l32;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(&lB[buf][r * kLdsRow + 32 * ks + 16 * h]);
        b[j] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        sb[j] = (int)((sB[buf][r] >> (8 * (2 * ks + h))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                      sb[j]);
    }
    if (st + 1 < nst) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * TN * 32 + j * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M && col < N) store_out(C + (int64_t)row * ldc + col, alpha * acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// Main path (K a multiple of 128): operands move from global memory straight
// into LDS (global_load_lds_dwordx4; lane l of a wave writes bytes
// [16 l, 16 l + 16) after the wave's LDS base) through a ring of NS stages,
// so that up to NS - 1 stages of loads are in flight while the matrix cores
// consume one.  Per stage a row contributes 64 bytes (four 16-byte chunks:
// 128 FP4 codes or 32 bf16 values) and, for MXFP4, one dword of E8M0 scales.
// Rows are stored unpadded, with chunk c of row r at position c ^ sw(r),
// sw(r) = (r >> 2) & 3.  This LDS serves a 16-byte read for 16 lanes per
// cycle from 64 banks; with this swizzle the 16 rows of each group fall on
// distinct banks, and the bank-conflict counter reads close to zero.  Rows
// past M or N are loaded from row M - 1 or N - 1 (no branches); they only
// feed outputs that are never stored.
template <int ROWB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (ROWB == 64) return (r >> 2) & 3;  // 16 rows of 64 B cover all 64 banks 4 times
  else return (r >> 1) & 7;                       // 128-byte rows: 8 chunks, rows pair up per bank half
}

// This lane's index in its wave, opaque to the optimiser (values derived from it are computed
// where they are used rather than hoisted out of loops).
__device__ __forceinline__ int opaque_lane() {
  int l = (int)(threadIdx.x & 63);
  __asm__ volatile("" : "+v"(l));
  return l;
}

// s_waitcnt with only the vector-memory counter (expcnt, lgkmcnt at their maxima)
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

__device__ __forceinline__ void load_lds16(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                   (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                   (__attribute__((address_space(3))) void *)l, 4, 0, 0);
}

// Whether one ring stage can hold the epilogue's staging area (the persistent form stages the
// output in the slot of a tile's last stage while the other slot holds the next tile's first).
template <int WGM, int WGN, int TM, int TN, typename OutT, bool MX, int ROWB>
constexpr bool ring_stage_holds_epilogue() {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32, SPR = ROWB / 16;
  constexpr int stage = MX ? (BM + BN) * (ROWB + SPR) : (BM + BN) * ROWB;
  constexpr int staging = WGM * WGN * 32 * (TN * 32 + 16 / (int)sizeof(OutT)) * (int)sizeof(OutT);
  return staging <= stage;
}

// Compute units of the current device (cached per device, safe to call from several host threads;
// 0 if the query fails).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int q = 0;
    if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && q > 0) {
      cache[dev].store(q, std::memory_order_relaxed);
      n = q;
    }
  }
  return n;
}

// LDS bytes of a ring kernel instantiation, and the workgroups of it one CU holds (160 KB of LDS
// per CU on gfx950; the ring kernels are LDS-bound in occupancy).
template <int WGM, int WGN, int TM, int TN, int NS, bool MX, int ROWB, bool SCALE16>
constexpr int ring_lds_bytes() {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32, SPR = ROWB / 16;
  constexpr int stage = MX ? (BM + BN) * (ROWB + SPR) : (BM + BN) * ROWB;
  return NS * stage + (SCALE16 ? 1024 : 256);
}
constexpr int kLdsPerCu = 160 * 1024;

// Grid of the persistent ring: as many workgroups as the CUs hold at once (per_cu each), a
// multiple of the XCD count so that the workgroup -> XCD assignment matches the tile order; 0 (use
// the one-tile form) when a product has no more tiles than that, or when an operand's rows (rows x
// row_bytes, row_bytes >= its scale bytes per row) reach 4 GiB, past the kernel's 32-bit load
// offsets.
int persistent_grid(int64_t tiles, int64_t rows, int64_t row_bytes, int per_cu) {
  if (rows * row_bytes + 4096 > (int64_t)UINT32_MAX) return 0;
  const int slots = device_cus() * per_cu;
  const int g = slots - slots % kXcds;
  return (g > 0 && tiles > g) ? g : 0;
}

// Where the E8M0 bytes of row r for stage st are: S + r * row + st * stage.  Row-major scales (the
// quantizer's layout): row = K / 32, stage = scale bytes per stage.  Stage-major scales
// ([K / (2 ROWB)][rows][ROWB / 16], written by the scale reorganisation pass): row = ROWB / 16,
// stage = rows * ROWB / 16, so one stage of a tile's scales is one contiguous run.
struct ScaleLayout {
  int64_t a_row, a_stage, b_row, b_stage;
};

// MX = true: MXFP4 operands (a stage is 2 ROWB K elements = ROWB code bytes + ROWB / 16 E8M0 bytes
// per row; v_mfma_scale_f32_32x32x64_f8f6f4).  K step ks of a stage (KS = ROWB / 32 steps) takes, in
// lane half h, the 32-element block h KS + ks of the stage, so that a lane's KS scale bytes of a
// stage are contiguous: they are read as one word per row per stage, and the MFMA's byte select
// (op_sel, checked on the device) picks byte ks.  MX = false: bf16 operands (a stage is 32 K elements = 64 bytes
// per row; v_mfma_f32_32x32x16_bf16, lane l holding row l % 32 and K elements 8 (l / 32) .. +8, checked
// on the device), scaled at the end by fp32(*ga * *gb).  Rows are kb bytes apart; nst stages.
template <int WGM, int WGN, int TM, int TN, int NS, typename OutT, bool MX = true, int ROWB = 64,
          bool SCALE16 = false, bool PERSIST = false>
__global__ __launch_bounds__(64 * WGM * WGN) void mx_gemm_ring_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, int M, int N, int nst, int64_t kb, ScaleLayout sl, const float *__restrict__ ga,
    const float *__restrict__ gb, float alpha, OutT *__restrict__ C, int64_t ldc) {
  constexpr int WAVES = WGM * WGN;
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  static_assert(ROWB == 64 || ROWB == 128, "a stage holds 64 or 128 bytes of each row");
  constexpr int CPR = ROWB / 16;  // 16-byte chunks per row per stage
  constexpr int KS = ROWB / 32;   // k steps per stage (32 bytes of a row each)
  constexpr int SPR = ROWB / 16;  // MXFP4 scale bytes per row per stage
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int SA_OFF = A_BYTES + B_BYTES, SB_OFF = SA_OFF + BM * SPR;
  constexpr int STAGE = MX ? SB_OFF + BN * SPR : A_BYTES + B_BYTES;
  // 1 KB code loads (1024 / ROWB rows each) and 256 B scale loads per stage, spread over the waves
  constexpr int RPL = 1024 / ROWB;
  constexpr int A_INSTR = BM / RPL / WAVES, B_INSTR = BN / RPL / WAVES;
  // scale loads: 256 B (4 bytes per lane, row-major scales) or, SCALE16, 1 KB (16 bytes per lane,
  // two rows of stage-major scales each)
  constexpr int SBYTES = SCALE16 ? 1024 : 256;
  constexpr int SA_INSTR = BM * SPR / SBYTES, SB_INSTR = BN * SPR / SBYTES;
  // every wave issues the same number of scale loads (a wave without one loads into a spare slot),
  // so that the per-wave count of loads per stage is a constant
  constexpr int SQ = MX ? (SA_INSTR + SB_INSTR + WAVES - 1) / WAVES : 0;
  static_assert(A_INSTR * WAVES * RPL == BM && B_INSTR * WAVES * RPL == BN, "code loads must divide evenly");
  static_assert(!MX || (SA_INSTR * SBYTES == BM * SPR && SB_INSTR * SBYTES == BN * SPR),
                "scale loads cover whole rows");
  static_assert(!SCALE16 || SPR == 8, "16-byte scale loads take two rows of 8 scale bytes");
  // PERSIST: the waits below are all vmcnt(0) only with two slots, which keeps them exact once
  // epilogue stores share the counter with the loads
  static_assert(!PERSIST || NS == 2, "the persistent form runs a two-slot ring");
  constexpr int LOADS = A_INSTR + B_INSTR + SQ;  // per wave per stage
  constexpr int SPARE = NS * STAGE;               // target of the filler scale loads
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE + SBYTES];
  if constexpr (!MX) alpha = (*ga) * (*gb);

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // Tiles of this workgroup.  One launch tile per workgroup, or (PERSIST, gridDim.x a multiple of
  // the XCD count) tiles blockIdx.x + j gridDim.x for j = 0, 1, ...: the tiles the one-per-workgroup
  // launch would give those workgroup ids, so each stays on the same XCD in the same round.
  const int total = PERSIST ? tiles_m * tiles_n : (int)gridDim.x;
  const int ntiles = PERSIST ? (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 1;
  // the wave index is the same in every lane of a wave: readfirstlane lets the compiler keep it and
  // what derives from it in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int l32 = lane & 31, h = lane >> 5;
  // split K (blockIdx.y, one tile per workgroup): this workgroup sums stages [sp nst, (sp + 1) nst)
  // into its own M x ldc partial (row-major scales only)
  if (!PERSIST && gridDim.y > 1) {
    const int64_t sp = blockIdx.y;
    A += sp * nst * ROWB;
    B += sp * nst * ROWB;
    As += sp * nst * sl.a_stage;
    Bs += sp * nst * sl.b_stage;
    C += sp * M * ldc;
  }

  // per-lane source addresses of the loads for the tile whose stages are being issued (advanced by
  // ROWB code bytes / SPR scale bytes per stage)
  // Sources of the loads, as byte offsets from the operand (A, B, As or Bs) of each load: 32-bit
  // per-lane offsets for PERSIST (every operand under 4 GiB: checked by the launch), which keeps
  // the register file free for the tile loop; 64-bit otherwise.
  using Off = std::conditional_t<PERSIST, uint32_t, int64_t>;
  Off offA[A_INSTR], offB[B_INSTR];
  // scale load q covers 256 bytes: 256 / SPR rows, lane l loading dword l % (SPR / 4) of row l / (SPR / 4)
  constexpr int DPR = SPR / 4;  // scale dwords per row per stage
  Off offS[SQ > 0 ? SQ : 1];
  const uint8_t *baseS[SQ > 0 ? SQ : 1];
  int64_t stepS[SQ > 0 ? SQ : 1];
  int dstS[SQ > 0 ? SQ : 1];
  auto set_sources = [&](int j) {
    const int lane = ::fp4q_gemm::opaque_lane();
    int tm, tn;
    tile_of((int)blockIdx.x + j * (int)gridDim.x, total, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int row = (wave * A_INSTR + i) * RPL + lane / CPR;
      offA[i] = (Off)((int64_t)min(m0 + row, M - 1) * kb + 16 * ((lane % CPR) ^ swz<ROWB>(row)));
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      const int row = (wave * B_INSTR + i) * RPL + lane / CPR;
      offB[i] = (Off)((int64_t)min(n0 + row, N - 1) * kb + 16 * ((lane % CPR) ^ swz<ROWB>(row)));
    }
#pragma unroll
    for (int j2 = 0; j2 < SQ; ++j2) {
      const int q = wave + WAVES * j2;
      // SCALE16: lane l loads rows 2l, 2l + 1 (16 contiguous bytes of stage-major scales); the row is
      // clamped to the last one, and a pair starting there reads 8 bytes past the rows' end (the
      // reorganised copy is padded for it)
      const int rl = SCALE16 ? 2 * lane : lane / DPR, dw = SCALE16 ? 0 : lane % DPR;
      constexpr int RPS = SBYTES / SPR;  // rows per scale load
      if (q < SA_INSTR) {
        baseS[j2] = As;
        offS[j2] = (Off)((int64_t)min(m0 + RPS * q + rl, M - 1) * sl.a_row + 4 * dw);
        stepS[j2] = sl.a_stage;
        dstS[j2] = SA_OFF + SBYTES * q;
      } else if (q < SA_INSTR + SB_INSTR) {
        const int qb = q - SA_INSTR;
        baseS[j2] = Bs;
        offS[j2] = (Off)((int64_t)min(n0 + RPS * qb + rl, N - 1) * sl.b_row + 4 * dw);
        stepS[j2] = sl.b_stage;
        dstS[j2] = SB_OFF + SBYTES * qb;
      } else {
        baseS[j2] = As;
        offS[j2] = (Off)((int64_t)min(m0 + rl, M - 1) * sl.a_row + 4 * dw);
        stepS[j2] = sl.a_stage;
        dstS[j2] = -1;
      }
    }
  };

  auto issue = [&](int st, int slot) {
    uint8_t *base = smem + slot * STAGE;
    const uint8_t *a_st = A + (int64_t)st * ROWB, *b_st = B + (int64_t)st * ROWB;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) load_lds16(a_st + offA[i], base + (wave * A_INSTR + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) load_lds16(b_st + offB[i], base + A_BYTES + (wave * B_INSTR + i) * 1024);
#pragma unroll
    for (int j = 0; j < SQ; ++j) {
      uint8_t *d = dstS[j] >= 0 ? base + dstS[j] : smem + SPARE;
      const uint8_t *src = baseS[j] + st * stepS[j] + offS[j];
      if constexpr (SCALE16) load_lds16(src, d);
      else load_lds4(src, d);
    }
  };
  // The issue stream runs over the stages of all this workgroup's tiles in order, NS stages ahead
  // of the MFMAs; past the last stage it reloads the last stage (never read again).  Every call
  // issues exactly one stage of loads, so each wait below is one constant.
  int iss_j = 0, iss_st = 0;
  set_sources(0);
  auto issue_next = [&](int slot) {
    issue(iss_j < ntiles ? iss_st : nst - 1, slot);
    if (iss_j < ntiles && ++iss_st == nst) {
      iss_st = 0;
      if (++iss_j < ntiles) set_sources(iss_j);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{0};

  // operands of one k step: code registers for TM blocks of A and TN of B, and (MX) the stage's
  // scale words
  struct Ops {
    i32x8 a[TM], b[TN];
    int sa[TM], sb[TN];
  };
  // LDS chunk (16 bytes) of k step ks in lane half h
  auto chunk = [&](int ks) { return MX ? h * KS + ks : 2 * ks + h; };
  auto scale_word = [&](const uint8_t *p) {
    if constexpr (SPR == 8) return (int)*reinterpret_cast<const uint32_t *>(p + 4 * h);
    else return (int)*reinterpret_cast<const uint16_t *>(p + 2 * h);
  };
  // The rows a lane reads are l32 plus multiples of 32, and swz looks only at bits 1-3 (or 2-3) of
  // the row, so every row this lane reads has its lane's swizzle: one per-lane offset per k step,
  // with the block offsets as immediates.
  const int lane_sw = swz<ROWB>(l32);
  auto read_ops = [&](int slot_, auto ks_c, Ops &o, const Ops &prev) {
    constexpr int ks = decltype(ks_c)::value;
    const uint8_t *base = smem + slot_ * STAGE + l32 * ROWB + 16 * (chunk(ks) ^ lane_sw);
    const uint8_t *base_a = base + wm * TM * 32 * ROWB, *base_b = base + A_BYTES + wn * TN * 32 * ROWB;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const i32x4 v = *reinterpret_cast<const i32x4 *>(base_a + i * 32 * ROWB);
      o.a[i] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
      if constexpr (MX)
        o.sa[i] = ks == 0 ? scale_word(smem + slot_ * STAGE + SA_OFF + SPR * (wm * TM * 32 + i * 32 + l32))
                          : prev.sa[i];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const i32x4 v = *reinterpret_cast<const i32x4 *>(base_b + j * 32 * ROWB);
      o.b[j] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
      if constexpr (MX)
        o.sb[j] = ks == 0 ? scale_word(smem + slot_ * STAGE + SB_OFF + SPR * (wn * TN * 32 + j * 32 + l32))
                          : prev.sb[j];
    }
  };
  auto mfmas = [&](const Ops &o, auto ks_c) {
    constexpr int ks = decltype(ks_c)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (MX) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[i], o.b[j], acc[i][j], 4, 4, ks, o.sa[i],
                                                                      ks, o.sb[j]);
        } else {
          const i32x4 av = {o.a[i][0], o.a[i][1], o.a[i][2], o.a[i][3]};
          const i32x4 bv = {o.b[j][0], o.b[j][1], o.b[j][2], o.b[j][3]};
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                              __builtin_bit_cast(bf16x8, bv), acc[i][j], 0, 0, 0);
        }
      }
  };
  // A barrier between stages: the compiler-only fences keep LDS reads on their side of it;
  // no workgroup fence, which would also drain the loads still in flight.
  auto stage_barrier = [&]() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // Epilogue staging: each wave writes one 32-row block of its tile at a time into its own LDS area
  // (row-major, padded), then stores it with 16-byte writes along the rows of C.  PERSIST stages in
  // the slot of the tile's last stage (the other slot holds the next tile's first stage).
  constexpr int WCOLS = TN * 32;                    // columns of a wave's tile
  constexpr int EPAD = 16 / (int)sizeof(OutT);      // 16 bytes of padding per row
  constexpr int EROW = WCOLS + EPAD;                // elements per staged row
  constexpr int VEC = 16 / (int)sizeof(OutT);       // elements per 16-byte store
  constexpr int LPR = WCOLS / VEC;                  // lanes per row
  constexpr int RPI = 64 / LPR;                     // rows per store instruction
  constexpr int EBYTES = WAVES * 32 * EROW * (int)sizeof(OutT);
  static_assert(EBYTES <= (PERSIST ? STAGE : NS * STAGE), "epilogue staging must fit in the ring");
  static_assert(!PERSIST || ring_stage_holds_epilogue<WGM, WGN, TM, TN, OutT, MX, ROWB>(), "staging size");
  const bool vec_ok = ((uintptr_t)C % 16 == 0) && ((ldc * (int64_t)sizeof(OutT)) % 16 == 0);
  auto epilogue = [&](int m0, int n0, uint8_t *area) {
    // lane-dependent addresses come from an opaque copy of the lane index, so that the compiler
    // computes them here instead of holding them in registers across the whole tile loop
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int l32 = ln & 31, h = ln >> 5;
    OutT *stage_out = reinterpret_cast<OutT *>(area) + wave * 32 * EROW;
    const int col0 = n0 + wn * WCOLS;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          // registers v and v + 1 hold rows r and r + 1 of the same column
          const int r = 8 * (v >> 2) + 4 * h + (v & 3);
          OutT *o = stage_out + r * EROW + j * 32 + l32;
          if constexpr (sizeof(OutT) == 4) {
            o[0] = alpha * acc[i][j][v];
            o[EROW] = alpha * acc[i][j][v + 1];
          } else {
            const uint32_t p = f32x2_to_bf16x2(alpha * acc[i][j][v], alpha * acc[i][j][v + 1]);
            o[0] = (uint16_t)p;
            o[EROW] = (uint16_t)(p >> 16);
          }
        }
      const int row0 = m0 + wm * TM * 32 + i * 32;
#pragma unroll
      for (int q = 0; q < 32 / RPI; ++q) {
        const int r = q * RPI + ln / LPR, c = (ln % LPR) * VEC;
        const int row = row0 + r, col = col0 + c;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(stage_out + r * EROW + c);
        if (row < M) {
          OutT *dst = C + (int64_t)row * ldc + col;
          if (vec_ok && col + VEC <= N) {
            *reinterpret_cast<i32x4 *>(dst) = v;
          } else {
            const OutT *e = reinterpret_cast<const OutT *>(&v);
#pragma unroll
            for (int t = 0; t < VEC; ++t)
              if (col + t < N) dst[t] = e[t];
          }
        }
      }
    }
  };

  // Stage g of the stream sits in slot g % NS.  Stages 0 .. NS-1 are issued up front; in the
  // iteration of stage g, once every wave has read all of it, stage g + NS is issued into its slot.
  // After stage g + 1 has landed, NS - 2 stages of this wave's loads may still be in flight.
  Ops o0, o1;
  int slot = 0;
  // k steps 0 .. KS-2 of the stage in `slot`: read step ks + 1 while step ks's MFMAs run (KS is even:
  // o0 holds the even steps), then wait until stage g + 1 has landed and every wave is past stage g
  // PERSIST: the MFMAs issued so far are placed here.  The compiler treats them as pure and would
  // otherwise sink them below later branches (the tile-boundary branch of the issue stream, the
  // epilogue's row blocks), past the barrier and with every k step's operands live at once.  The
  // empty asm emits nothing.
  auto pin_acc = [&]() {
    if constexpr (PERSIST) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) __asm__ volatile("" : "+v"(acc[i][j]));
    }
  };
  auto stage_body = [&]() {
    unroll(std::make_integer_sequence<int, KS - 1>{}, [&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      if constexpr (ks % 2 == 0) {
        read_ops(slot, std::integral_constant<int, ks + 1>{}, o1, o0);
        mfmas(o0, ks_c);
      } else {
        read_ops(slot, std::integral_constant<int, ks + 1>{}, o0, o1);
        mfmas(o1, ks_c);
      }
    });
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);  // keep these MFMAs ahead of the barrier below
    wait_lgkmcnt0();                    // this wave's reads of stage g are complete
    wait_vmcnt<(NS - 2) * LOADS>();     // stage g + 1 has landed
    stage_barrier();                    // ... for every wave, and nobody reads stage g any more
  };
  if constexpr (!PERSIST) {
    // one tile: past the last stage every iteration reloads the last stage into the slot just freed
#pragma unroll
    for (int s = 0; s < NS; ++s) issue(min(s, nst - 1), s);
    wait_vmcnt<(NS - 1) * LOADS>();
    stage_barrier();
    read_ops(0, std::integral_constant<int, 0>{}, o0, o1);
    for (int st = 0; st < nst; ++st) {
      stage_body();
      const int next = slot == NS - 1 ? 0 : slot + 1;
      issue(min(st + NS, nst - 1), slot);
      read_ops(next, std::integral_constant<int, 0>{}, o0, o1);  // the next stage's first k step
      __builtin_amdgcn_sched_barrier(0);
      mfmas(o1, std::integral_constant<int, KS - 1>{});
      slot = next;
    }
    int tm, tn;
    tile_of(blockIdx.x, total, tiles_m, tiles_n, tm, tn);
    __syncthreads();  // every wave is done reading the ring
    epilogue(tm * BM, tn * BN, smem);
  } else {
    // The issue stream continues from one tile into the next.  A tile's last stage is peeled: its
    // issue waits until the epilogue has staged the output through that stage's slot (the other
    // slot already holds the next tile's first stage), and a tile with no successor issues nothing
    // more.  Every wait is vmcnt(0) (two slots), so the epilogue's stores in the counter are waited
    // for with the loads.
#pragma unroll
    for (int s = 0; s < NS; ++s) issue_next(s);
    wait_vmcnt<(NS - 1) * LOADS>();
    stage_barrier();
    read_ops(0, std::integral_constant<int, 0>{}, o0, o1);
#pragma nounroll
    for (int j = 0; j < ntiles; ++j) {
#pragma nounroll
      for (int st = 0; st + 1 < nst; ++st) {
        stage_body();
        const int next = slot == NS - 1 ? 0 : slot + 1;
        issue_next(slot);
        read_ops(next, std::integral_constant<int, 0>{}, o0, o1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(o1, std::integral_constant<int, KS - 1>{});
        slot = next;
      }
      stage_body();
      mfmas(o1, std::integral_constant<int, KS - 1>{});
      pin_acc();
      int tm, tn;
      tile_of((int)blockIdx.x + j * (int)gridDim.x, total, tiles_m, tiles_n, tm, tn);
      epilogue(tm * BM, tn * BN, smem + slot * STAGE);
      const int next = slot == NS - 1 ? 0 : slot + 1;
      if (j + 1 < ntiles) {
        wait_lgkmcnt0();  // this wave's staging reads are complete
        stage_barrier();  // ... for every wave: the slot may be refilled
        issue_next(slot);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j2 = 0; j2 < TN; ++j2) acc[i][j2] = f32x16{0};
        read_ops(next, std::integral_constant<int, 0>{}, o0, o1);
      }
      slot = next;
    }
  }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

template <int TM, int TN, typename OutT>
hipError_t launch(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int m, int n, int k,
                  float alpha, OutT *c, int64_t ldc, hipStream_t s) {
  constexpr int BM = 2 * TM * 32, BN = 2 * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const bool dword = (k / 32) % 4 == 0 && aligned(as, 4) && aligned(bs, 4);
  if (dword)
    hipLaunchKernelGGL((mx_gemm_kernel<TM, TN, true, OutT>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a, as, b,
                       bs, m, n, k, alpha, c, ldc);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<TM, TN, false, OutT>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a, as,
                       b, bs, m, n, k, alpha, c, ldc);
  return hipGetLastError();
}

// MXFP4 operands; k a multiple of 2 * ROWB (a stage holds ROWB code bytes = 2 * ROWB elements per
// row).  staged: the scales were reorganised stage-major (as / bs point into that copy).  splits > 1
// (row-major scales, k a multiple of 2 ROWB splits): split j writes its partial sum over the j-th
// K range to c + j m ldc.
template <int WGM, int WGN, int TM, int TN, int NS, typename OutT, int ROWB = 64, bool SCALE16 = false>
hipError_t launch_ring(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int m, int n, int k,
                       float alpha, OutT *c, int64_t ldc, hipStream_t s, bool staged = false, int splits = 1) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int SPR = ROWB / 16;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const ScaleLayout sl = staged ? ScaleLayout{SPR, (int64_t)m * SPR, SPR, (int64_t)n * SPR}
                                : ScaleLayout{k / 32, SPR, k / 32, SPR};
  if constexpr (NS == 2 && ring_stage_holds_epilogue<WGM, WGN, TM, TN, OutT, true, ROWB>()) {
    // more tiles than CUs: one persistent workgroup per CU walks its tiles, fetching the next
    // tile's first stage while it finishes the current one
    constexpr int per_cu = kLdsPerCu / ring_lds_bytes<WGM, WGN, TM, TN, NS, true, ROWB, SCALE16>();
    const int grid = splits == 1 ? persistent_grid(tiles, std::max(m, n), k / 2, per_cu) : 0;
    if (grid > 0) {
      hipLaunchKernelGGL((mx_gemm_ring_kernel<WGM, WGN, TM, TN, NS, OutT, true, ROWB, SCALE16, true>), dim3(grid),
                         dim3(64 * WGM * WGN), 0, s, a, as, b, bs, m, n, k / (2 * ROWB), (int64_t)(k / 2), sl,
                         (const float *)nullptr, (const float *)nullptr, alpha, c, ldc);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mx_gemm_ring_kernel<WGM, WGN, TM, TN, NS, OutT, true, ROWB, SCALE16>),
                     dim3((unsigned)tiles, (unsigned)splits), dim3(64 * WGM * WGN), 0, s, a, as, b, bs, m, n,
                     k / (2 * ROWB) / splits, (int64_t)(k / 2), sl, (const float *)nullptr, (const float *)nullptr,
                     alpha, c, ldc);
  return hipGetLastError();
}

// Few-token product, M <= 16: one workgroup per 16 NT output columns, its W waves splitting K into
// contiguous ranges of S steps of 128 elements (W S 128 = K).  v_mfma_scale_f32_16x16x128_f8f6f4
// takes from lane l row l % 16 and the 32 elements at 32 (l / 16) of a step, and its accumulator
// register v of lane l holds row 4 (l / 16) + v, column l % 16 (both checked on the device).  Step s
// of a wave covers 128 contiguous elements of each row, so the four lanes of a row read 64
// contiguous code bytes per load; a row's scale bytes for four steps arrive in one 16-byte load, and
// lane l takes byte l / 16 of the step's word by a shift.  Every load is issued before the first
// MFMA (the whole product's bytes are in flight at once); the NT column tiles of a workgroup share
// one read of A.  The waves' sums meet in LDS and are added in ascending K order.
template <int S, int NT, int RT, typename OutT>
__global__ __launch_bounds__(1024) void mx_gemm_skinny_kernel(const uint8_t *__restrict__ A,
                                                              const uint8_t *__restrict__ As,
                                                              const uint8_t *__restrict__ B,
                                                              const uint8_t *__restrict__ Bs, int M, int N, int K,
                                                              float alpha, OutT *__restrict__ C, int64_t ldc) {
  static_assert(S % 4 == 0 && S <= 8 && NT >= 1 && NT <= 2 && RT >= 1 && RT * S <= 16 && (NT == 1 || RT == 1),
                "steps per wave, column tiles, row tiles");
  __shared__ float part[RT * NT][16][64][4];  // [row tile, column tile][wave][lane][register]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16 * NT;
  const int r16 = lane & 15, h = lane >> 4;
  const int kw0 = wave * S * 128;  // this wave's first K element
  const int64_t kb = K / 2, sb = K / 32;
  // rows past M repeat row M - 1: computed, never stored
  int arow[RT], brow[NT];
#pragma unroll
  for (int r = 0; r < RT; ++r) arow[r] = min(16 * r + r16, M - 1);
#pragma unroll
  for (int t = 0; t < NT; ++t) brow[t] = min(n0 + 16 * t + r16, N - 1);
  // every load is issued before the first MFMA, in the order of use: the scale words (16 bytes per
  // four steps), then step by step the codes of A and B, so that the first steps can start while
  // the later loads are in flight
  i32x4 bc[NT][S], ac[RT][S], bsw[NT][S / 4], asw[RT][S / 4];
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {  // scale bytes of steps 4q .. 4q+3 (blocks 4 step + h)
#pragma unroll
    for (int r = 0; r < RT; ++r)
      asw[r][q] = *reinterpret_cast<const i32x4 *>(As + (int64_t)arow[r] * sb + kw0 / 32 + 16 * q);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bsw[t][q] = *reinterpret_cast<const i32x4 *>(Bs + (int64_t)brow[t] * sb + kw0 / 32 + 16 * q);
  }
  __builtin_amdgcn_sched_barrier(0);
  unroll(std::make_integer_sequence<int, S>{}, [&](auto st_c) {
    constexpr int st = decltype(st_c)::value;
#pragma unroll
    for (int r = 0; r < RT; ++r)
      ac[r][st] = *reinterpret_cast<const i32x4 *>(A + (int64_t)arow[r] * kb + kw0 / 2 + 16 * h + 64 * st);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bc[t][st] = *reinterpret_cast<const i32x4 *>(B + (int64_t)brow[t] * kb + kw0 / 2 + 16 * h + 64 * st);
    __builtin_amdgcn_sched_barrier(0);
  });
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  f32x4v acc[RT][NT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  unroll(std::make_integer_sequence<int, S>{}, [&](auto st_c) {
    constexpr int st = decltype(st_c)::value;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const i32x8 a = {ac[r][st][0], ac[r][st][1], ac[r][st][2], ac[r][st][3], 0, 0, 0, 0};
      const int sa = (int)((uint32_t)asw[r][st / 4][st % 4] >> (8 * h));  // byte 0: block 4 st + h
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const i32x8 b = {bc[t][st][0], bc[t][st][1], bc[t][st][2], bc[t][st][3], 0, 0, 0, 0};
        const int sbv = (int)((uint32_t)bsw[t][st / 4][st % 4] >> (8 * h));
        acc[r][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[r][t], 4, 4, 0, sa, 0, sbv);
      }
    }
  });
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[r * NT + t][wave][lane][v] = acc[r][t][v];
  __syncthreads();
  for (int i = threadIdx.x; i < 256 * RT * NT; i += blockDim.x) {
    const int rt = i >> 8, t = rt % NT, m = 16 * (rt / NT) + ((i >> 4) & 15), j = i & 15;
    const int l = 16 * ((m & 15) >> 2) + j, v = m & 3;  // the lane and register holding (m, j)
    float sum = part[rt][0][l][v];
    for (int w = 1; w < waves; ++w) sum = sum + part[rt][w][l][v];
    const int col = n0 + 16 * t + j;
    if (m < M && col < N) store_out(C + (int64_t)m * ldc + col, alpha * sum);
  }
}

// Column tiles per workgroup of the few-token kernel: two (one read of A serves 32 columns) for more
// than one token once the output is wide enough to keep the chip busy with half as many
// workgroups; past 16384 columns one tile measured faster up to eight tokens.
int skinny_tiles(int64_t m, int64_t n) { return (m > 1 && n >= 8192 && (n <= 16384 || m > 8)) ? 2 : 1; }

// Steps per wave of the few-token kernel for this shape, or 0 when it does not apply: M above 64, K
// not a multiple of 512, or no S in {4, 8} with W = K / (128 S) <= 16 waves.  Beyond one 16-row tile
// (M > 16) only S = 4 (K <= 8192): two row tiles of eight steps measured slower than the split.
int skinny_steps(int64_t m, int64_t k) {
  if (m > 64 || m <= 0 || k % 512) return 0;
  const int64_t nst = k / 128;
  for (int S : {4, 8})
    if (nst % S == 0 && nst / S <= 16) return (m <= 16 || S == 4) ? S : 0;
  return 0;
}

// ---------------------------------------------------------------- few-token NVFP4 product ------
// An E4M3 block scale V splits into a power of two 2^e and a significand m (V = 2^e m): normal
// patterns 2^(E-7) and 1 + F/8, subnormal ones 2^-9 and F, with the sign on m; NaN patterns give
// m = NaN, and zero m = 0.  The scaled FP4 convert applies only the exponent of its scale operand
// (checked on the device), so it yields q 2^e exactly in float16, and one packed float16 multiply
// by m makes q V, exact as well: q has two significant bits and m four, and |q V| lies in
// [2^-10, 2688], inside float16's normal range.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 nv_scale_parts(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, f = b & 7u;
  uint32_t p2, m;
  if (e == 15u && f == 7u) {
    p2 = 0x3F800000u;  // 1.0
    m = 0x7E00u;       // NaN
  } else if (e == 0u) {
    p2 = 118u << 23;  // 2^-9
    m = __builtin_bit_cast(uint16_t, (_Float16)(float)f);
  } else {
    p2 = (e + 120u) << 23;  // 2^(E-7)
    m = 0x3C00u | (f << 7);  // 1 + F/8
  }
  m |= (b & 0x80u) << 8;
  return make_uint2(p2, m | (m << 16));
}

// Eight consecutive FP4 codes (one dword) times the block scale held in parts (p2, m2).
__device__ __forceinline__ f16x8 nv_decode8(uint32_t dw, uint2 parts) {
  const float p2 = __uint_as_float(parts.x);
  const f16x2 m = __builtin_bit_cast(f16x2, parts.y);
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, p2, 0) * m;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, p2, 1) * m;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, p2, 2) * m;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, p2, 3) * m;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Scale byte of lane quarter h for group g, half i of its 32 elements, out of the 16-byte loads
// v[] holding a row's scale bytes of the wave's range (8 per 128-element group).
template <int G, int I>
__device__ __forceinline__ uint32_t nv_scale_byte(const i32x4 *v, int h) {
  constexpr int q = G / 2, d = 2 * (G % 2);
  const uint32_t w = (uint32_t)((h & 2) ? v[q][d + 1] : v[q][d]);
  return (w >> (8 * (2 * (h & 1) + I))) & 0xFFu;
}

// Few-token NVFP4 product, M <= 16: one workgroup per 16 NT output columns, its W waves splitting K
// into contiguous ranges of S groups of 128 elements (W S 128 = K).  In group g, lane l (row l % 16,
// quarter h = l / 16) holds the 32 elements at 128 g + 32 h of its row (one 16-byte load; the four
// lanes of a row read 64 contiguous bytes) and feeds them to four v_mfma_f32_16x16x32_f16 steps,
// eight at a time (step s: elements 8 s .. 8 s + 7 of every lane, in both operands alike).  Every
// code and scale load is issued before the first decode, in the order of use.  The accumulator's
// register v of lane l holds row 4 (l / 16) + v, column l % 16; the waves' sums meet in LDS, are
// added in ascending K order and scaled by fp32(S_a S_b).  The small variants are held to 64 VGPRs,
// so that two 16-wave workgroups fit on a CU.
template <int S, int NT, int RT, bool SEG, typename OutT>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(S * NT * RT <= 4 ? 8 : 4))) void
nv_gemm_skinny_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
                      const uint8_t *__restrict__ Bs, int M, int N, int K, const float *__restrict__ ga,
                      const float *__restrict__ gb, OutT *__restrict__ C, int64_t ldc, float *__restrict__ P) {
  static_assert(S % 2 == 0 && S <= 8 && NT >= 1 && NT <= 2 && RT >= 1 && RT * S <= 8 && (NT == 1 || RT == 1),
                "groups per wave, column tiles, row tiles");
  __shared__ float part[RT * NT][16][64][4];  // [row tile, column tile][wave][lane][register]
  __shared__ uint2 scale_parts[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16 * NT;
  const int r16 = lane & 15, h = lane >> 4;
  // SEG: K in gridDim.y contiguous segments; workgroup y takes the y-th and writes its unscaled sums
  // to P[y] (M x N), added in K order by the split sum kernel
  const int kw0 = (SEG ? blockIdx.y * waves * S * 128 : 0) + wave * S * 128;  // this wave's first K element
  const int64_t kb = K / 2, sb = K / 16;
  // rows past M repeat row M - 1 (and columns past N column N - 1): computed, never stored
  int arow[RT], brow[NT];
#pragma unroll
  for (int r = 0; r < RT; ++r) arow[r] = min(16 * r + r16, M - 1);
#pragma unroll
  for (int t = 0; t < NT; ++t) brow[t] = min(n0 + 16 * t + r16, N - 1);
  // every load first, in the order of use: scale bytes (16 bytes per two groups), then group by group
  // the codes of A and B (one 16-byte load each), so the first groups' decode overlaps the rest
  i32x4 bc[NT][S], ac[RT][S], bsv[NT][S / 2], asv[RT][S / 2];
#pragma unroll
  for (int q = 0; q < S / 2; ++q) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
      asv[r][q] = *reinterpret_cast<const i32x4 *>(As + (int64_t)arow[r] * sb + kw0 / 16 + 16 * q);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bsv[t][q] = *reinterpret_cast<const i32x4 *>(Bs + (int64_t)brow[t] * sb + kw0 / 16 + 16 * q);
  }
  __builtin_amdgcn_sched_barrier(0);
  unroll(std::make_integer_sequence<int, S>{}, [&](auto g_c) {
    constexpr int g = decltype(g_c)::value;
#pragma unroll
    for (int r = 0; r < RT; ++r)
      ac[r][g] = *reinterpret_cast<const i32x4 *>(A + (int64_t)arow[r] * kb + kw0 / 2 + 16 * h + 64 * g);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bc[t][g] = *reinterpret_cast<const i32x4 *>(B + (int64_t)brow[t] * kb + kw0 / 2 + 16 * h + 64 * g);
    __builtin_amdgcn_sched_barrier(0);
  });
  for (int i = threadIdx.x; i < 256; i += blockDim.x) scale_parts[i] = nv_scale_parts((uint32_t)i);
  __syncthreads();
  f32x4 acc[RT][NT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  unroll(std::make_integer_sequence<int, S>{}, [&](auto g_c) {
    constexpr int g = decltype(g_c)::value;
    uint2 sap[RT][2], sbp[NT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      sap[r][0] = scale_parts[nv_scale_byte<g, 0>(asv[r], h)];
      sap[r][1] = scale_parts[nv_scale_byte<g, 1>(asv[r], h)];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sbp[t][0] = scale_parts[nv_scale_byte<g, 0>(bsv[t], h)];
      sbp[t][1] = scale_parts[nv_scale_byte<g, 1>(bsv[t], h)];
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f16x8 b[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) b[t] = nv_decode8((uint32_t)bc[t][g][st], st < 2 ? sbp[t][0] : sbp[t][1]);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const f16x8 a = nv_decode8((uint32_t)ac[r][g][st], st < 2 ? sap[r][0] : sap[r][1]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[r][t], 0, 0, 0);
      }
    }
  });
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[r * NT + t][wave][lane][v] = acc[r][t][v];
  __syncthreads();
  const float alpha = SEG ? 1.0f : (*ga) * (*gb);
  for (int i = threadIdx.x; i < 256 * RT * NT; i += blockDim.x) {
    const int rt = i >> 8, t = rt % NT, m = 16 * (rt / NT) + ((i >> 4) & 15), j = i & 15;
    const int l = 16 * ((m & 15) >> 2) + j, v = m & 3;  // the lane and register holding (m, j)
    float sum = part[rt][0][l][v];
    for (int w = 1; w < waves; ++w) sum = sum + part[rt][w][l][v];
    const int col = n0 + 16 * t + j;
    if (m < M && col < N) {
      if constexpr (SEG) P[((int64_t)blockIdx.y * M + m) * N + col] = sum;
      else store_out(C + (int64_t)m * ldc + col, alpha * sum);
    }
  }
}

// Plan of the few-token NVFP4 kernel: S groups of 128 elements per wave and KS segments of K (one
// workgroup each, partial sums in the workspace), or S = 0 when it does not apply: M above 32 (64
// for outputs of at most 4096 columns; wider ones ran faster tiled from three row tiles on), K not a
// multiple of 256, or no S in {2, 4, 8} with RT S <= 8 (RT = ceil(M / 16) row tiles) and at most 16
// waves of S groups per segment, KS in {1, 2, 4}.
struct NvSkinnyPlan {
  int S, KS;
};
NvSkinnyPlan nv_skinny_plan(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || m > 64 || (m > 32 && n > 4096) || k % 256) return {0, 1};
  const int64_t ng = k / 128, rt = (m + 15) / 16;
  for (int KS : {1, 2, 4})
    for (int S : {2, 4, 8})
      if (rt * S <= 8 && ng % ((int64_t)S * KS) == 0 && ng / ((int64_t)S * KS) <= 16) return {S, KS};
  return {0, 1};
}

// C = alpha * (P_0 + P_1 + ... + P_{splits-1}), the split partial sums added in ascending K order
// (splits <= kMaxSplits).  Row blockIdx.y, columns from blockIdx.x; every partial is loaded before
// the first addition, so the loads overlap.
constexpr int kMaxSplits = 16;
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ P, int splits, int m, int n,
                                                         float alpha, const float *__restrict__ ga,
                                                         const float *__restrict__ gb, OutT *__restrict__ C,
                                                         int64_t ldc) {
  const int col = blockIdx.x * 256 + threadIdx.x, r = blockIdx.y;
  if (col >= n) return;
  if (ga) alpha = (*ga) * (*gb);  // NVFP4: fp32(S_a S_b)
  const int64_t plane = (int64_t)m * n, t = (int64_t)r * n + col;
  float v[kMaxSplits];
#pragma unroll
  for (int j = 0; j < kMaxSplits; ++j) v[j] = j < splits ? P[j * plane + t] : 0.0f;
  float acc = v[0];
#pragma unroll
  for (int j = 1; j < kMaxSplits; ++j)
    if (j < splits) acc = acc + v[j];
  store_out(C + (int64_t)r * ldc + col, alpha * acc);
}

template <typename OutT>
hipError_t launch_nv_skinny(const uint8_t *a, const uint8_t *as, const float *ga, const uint8_t *b,
                            const uint8_t *bs, const float *gb, int m, int n, int k, NvSkinnyPlan plan, OutT *c,
                            int64_t ldc, float *parts, hipStream_t s) {
  const int S = plan.S, KS = plan.KS;
  const int rt = (m + 15) / 16;
  const int nt = rt == 1 && KS == 1 && skinny_tiles(m, n) == 2 && S <= 4 ? 2 : 1;
  const dim3 grid((unsigned)((n + 16 * nt - 1) / (16 * nt)), (unsigned)KS), block(64 * (k / (128 * S * KS)));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a, as, b, bs, m, n, k, ga, gb, c, ldc, parts);
  };
  auto pick = [&](auto seg_c) {
    constexpr bool SEG = decltype(seg_c)::value;
    if (S == 2) {
      if (rt == 1)
        nt == 1 ? go(nv_gemm_skinny_kernel<2, 1, 1, SEG, OutT>) : go(nv_gemm_skinny_kernel<2, 2, 1, SEG, OutT>);
      else if (rt == 2) go(nv_gemm_skinny_kernel<2, 1, 2, SEG, OutT>);
      else if (rt == 3) go(nv_gemm_skinny_kernel<2, 1, 3, SEG, OutT>);
      else go(nv_gemm_skinny_kernel<2, 1, 4, SEG, OutT>);
    } else if (S == 4) {
      if (rt == 1)
        nt == 1 ? go(nv_gemm_skinny_kernel<4, 1, 1, SEG, OutT>) : go(nv_gemm_skinny_kernel<4, 2, 1, SEG, OutT>);
      else go(nv_gemm_skinny_kernel<4, 1, 2, SEG, OutT>);
    } else {
      go(nv_gemm_skinny_kernel<8, 1, 1, SEG, OutT>);
    }
  };
  if (KS > 1) pick(std::true_type{});
  else pick(std::false_type{});
  if (KS > 1)
    hipLaunchKernelGGL((splitk_sum_kernel<OutT>), dim3((unsigned)((n + 255) / 256), (unsigned)m), dim3(256), 0, s,
                       (const float *)parts, KS, m, n, 1.0f, ga, gb, c, ldc);
  return hipGetLastError();
}

// bf16 operands (rows of kp elements, kp a multiple of ROWB / 2) scaled by fp32(*ga * *gb)
template <int WGM, int WGN, int TM, int TN, int NS, typename OutT, int ROWB = 64>
hipError_t launch_ring_bf16(const uint16_t *a, const uint16_t *b, int m, int n, int kp, const float *ga,
                            const float *gb, OutT *c, int64_t ldc, hipStream_t s) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if constexpr (NS == 2 && ring_stage_holds_epilogue<WGM, WGN, TM, TN, OutT, false, ROWB>()) {
    constexpr int per_cu = kLdsPerCu / ring_lds_bytes<WGM, WGN, TM, TN, NS, false, ROWB, false>();
    const int grid = persistent_grid(tiles, std::max(m, n), (int64_t)kp * 2, per_cu);
    if (grid > 0) {
      hipLaunchKernelGGL((mx_gemm_ring_kernel<WGM, WGN, TM, TN, NS, OutT, false, ROWB, false, true>), dim3(grid),
                         dim3(64 * WGM * WGN), 0, s, (const uint8_t *)a, (const uint8_t *)nullptr,
                         (const uint8_t *)b, (const uint8_t *)nullptr, m, n, kp * 2 / ROWB, (int64_t)kp * 2,
                         ScaleLayout{0, 0, 0, 0}, ga, gb, 1.0f, c, ldc);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mx_gemm_ring_kernel<WGM, WGN, TM, TN, NS, OutT, false, ROWB>), dim3((unsigned)tiles),
                     dim3(64 * WGM * WGN), 0, s, (const uint8_t *)a, (const uint8_t *)nullptr, (const uint8_t *)b,
                     (const uint8_t *)nullptr, m, n, kp * 2 / ROWB, (int64_t)kp * 2, ScaleLayout{0, 0, 0, 0}, ga, gb,
                     1.0f, c, ldc);
  return hipGetLastError();
}

// Scale reorganisation ("3. QuTLASS" of the MR-GPTQ page reorganises scales for its FP4 product):
// row-major E8M0 bytes [rows][k / 32] -> stage-major [k / 256][rows][8], so that the product's
// per-stage scale loads read contiguous runs instead of 8 bytes per row.  One launch covers both
// operands; a workgroup moves 64 rows x up to 64 stages through LDS, reading 8-byte pieces along
// rows and writing them along stages, both coalesced.
constexpr int kReoRows = 64, kReoStages = 64;

__global__ __launch_bounds__(256) void scales_to_stage_major_kernel(const uint8_t *__restrict__ sa, int ra,
                                                                    const uint8_t *__restrict__ sb, int rb, int k,
                                                                    int blocks_a, uint8_t *__restrict__ da,
                                                                    uint8_t *__restrict__ db) {
  __shared__ uint2 tile[kReoStages][kReoRows];
  const int stages = k / 256;
  const int chunks = (stages + kReoStages - 1) / kReoStages;
  const bool is_a = (int)blockIdx.x < blocks_a;
  const int b = is_a ? blockIdx.x : blockIdx.x - blocks_a;
  const uint8_t *src = is_a ? sa : sb;
  uint8_t *dst = is_a ? da : db;
  const int rows = is_a ? ra : rb;
  const int r0 = (b / chunks) * kReoRows, s0 = (b % chunks) * kReoStages;
  const int nr = min(kReoRows, rows - r0), ns = min(kReoStages, stages - s0);
  for (int e = threadIdx.x; e < nr * ns; e += 256) {
    const int r = e / ns, st = e % ns;
    tile[st][r] = *reinterpret_cast<const uint2 *>(src + (int64_t)(r0 + r) * (k / 32) + 8 * (s0 + st));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nr * ns; e += 256) {
    const int st = e / nr, r = e % nr;
    *reinterpret_cast<uint2 *>(dst + ((int64_t)(s0 + st) * rows + r0 + r) * 8) = tile[st][r];
  }
}

// (m + n) rows of k / 32 scale bytes, plus 16 bytes read past the end by a clamped 16-byte scale load
// K splits for a few-token product (M <= 64, whose 64 x 64 tiles alone would leave CUs idle): about
// one workgroup per CU (a narrower product already fills the chip and is not split: measured), the
// split partials (written and read once, 8 M N bytes per split) at most a quarter of B's code bytes
// (N K / 2), and a whole number of 128-byte stages per split, at least four (the depth of the load
// ring).
int gemm_mxfp4_splits(int64_t m, int64_t n, int64_t k) {
  if (m > 64 || m <= 0 || n <= 0 || k % 256) return 1;
  const int64_t tiles = (n + 63) / 64, nst = k / 256;
  const int64_t want = std::min<int64_t>(std::min<int64_t>(256 / tiles, nst / 4), std::max<int64_t>(1, k / (64 * m)));
  int best = 1;
  for (int64_t d = 2; d <= want && d <= nst && d <= kMaxSplits; ++d)
    if (nst % d == 0) best = (int)d;
  return best;
}

int64_t gemm_mxfp4_workspace(int64_t m, int64_t n, int64_t k) {
  if (k % 256) return 0;
  const int splits = gemm_mxfp4_splits(m, n, k);
  const int64_t reorg = (m + n) * (k / 32) + 32;
  return splits > 1 ? std::max<int64_t>(reorg, (int64_t)splits * m * n * 4) : reorg;
}

template <typename OutT>
hipError_t dispatch(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int m, int n, int k,
                    float alpha, OutT *c, int64_t ldc, hipStream_t s, uint8_t *ws = nullptr) {
  const int64_t big = (int64_t)((m + 255) / 256) * ((n + 255) / 256);
  const int64_t mid = (int64_t)((m + 127) / 128) * ((n + 127) / 128);
  // at most 16 tokens: the few-token kernel (whole K in flight, no workspace)
  // up to 16 tokens, or up to 64 when the output has at most 4096 columns (one workgroup per CU or
  // fewer; wider outputs ran faster on the tiled paths): the few-token kernel (whole K in flight, no
  // workspace)
  const int S = skinny_steps(m, k);
  if (S && (m <= 16 || n <= 4096) && aligned(as, 16) && aligned(bs, 16)) {
    const int waves = k / (128 * S);
    const int rt = (m + 15) / 16, nt = rt == 1 ? skinny_tiles(m, n) : 1;
    const dim3 grid((unsigned)((n + 16 * nt - 1) / (16 * nt))), block(64 * waves);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, a, as, b, bs, m, n, k, alpha, c, ldc); };
    if (S == 4) {
      if (rt == 1) nt == 1 ? go(mx_gemm_skinny_kernel<4, 1, 1, OutT>) : go(mx_gemm_skinny_kernel<4, 2, 1, OutT>);
      else if (rt == 2) go(mx_gemm_skinny_kernel<4, 1, 2, OutT>);
      else if (rt == 3) go(mx_gemm_skinny_kernel<4, 1, 3, OutT>);
      else go(mx_gemm_skinny_kernel<4, 1, 4, OutT>);
    } else {
      nt == 1 ? go(mx_gemm_skinny_kernel<8, 1, 1, OutT>) : go(mx_gemm_skinny_kernel<8, 2, 1, OutT>);
    }
    return hipGetLastError();
  }
  const int splits = gemm_mxfp4_splits(m, n, k);
  if (ws && splits > 1 && aligned(as, 4) && aligned(bs, 4)) {
    // few tokens: K split over workgroups, partial sums in the workspace, then added in K order
    float *parts = reinterpret_cast<float *>(ws);
    hipError_t e = launch_ring<2, 2, 1, 1, 4, float, 128>(a, as, b, bs, m, n, k, 1.0f, parts, n, s, false, splits);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((splitk_sum_kernel<OutT>), dim3((unsigned)((n + 255) / 256), (unsigned)m), dim3(256), 0, s,
                       parts, splits, m, n, alpha, (const float *)nullptr, (const float *)nullptr, c, ldc);
    return hipGetLastError();
  }
  const int64_t reo_blocks = ((m + kReoRows - 1) / kReoRows + (n + kReoRows - 1) / kReoRows) *
                             ((k / 256 + kReoStages - 1) / kReoStages);
  if (ws && k % 256 == 0 && big >= 256 && aligned(as, 8) && aligned(bs, 8) && reo_blocks < ((int64_t)1 << 31)) {
    // 256 x 256 tiles: reorganise both operands' scales stage-major first, so that each stage's scales
    // arrive in 1 KB loads (for smaller tiles the extra pass costs more than it saves: measured)
    uint8_t *was = ws, *wbs = ws + (int64_t)m * (k / 32) + 16;
    const int chunks = (k / 256 + kReoStages - 1) / kReoStages;
    const int blocks_a = (m + kReoRows - 1) / kReoRows * chunks, blocks_b = (n + kReoRows - 1) / kReoRows * chunks;
    hipLaunchKernelGGL(scales_to_stage_major_kernel, dim3(blocks_a + blocks_b), dim3(256), 0, s, as, m, bs, n, k,
                       blocks_a, was, wbs);
    return launch_ring<2, 4, 4, 2, 2, OutT, 128, true>(a, was, b, wbs, m, n, k, alpha, c, ldc, s, true);
  }
  // direct-to-LDS ring: 256 x 256 tiles when they give every CU a workgroup, 128 x 128 down to half
  // the CUs (two slots, so that two workgroups share a CU: measured 11-16% faster than three slots
  // and one), 64 x 64 for few-token products; stages of 128 code bytes per row (full 128-byte lines
  // per load) when K allows, else 64
  if (k % 256 == 0 && aligned(as, 4) && aligned(bs, 4)) {
    if (big >= 256) return launch_ring<2, 4, 4, 2, 2, OutT, 128>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
    if (mid >= 128) return launch_ring<2, 2, 2, 2, 2, OutT, 128>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
    return launch_ring<2, 2, 1, 1, 4, OutT, 128>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
  }
  if (k % 128 == 0 && aligned(as, 4) && aligned(bs, 4)) {
    if (big >= 256) return launch_ring<2, 4, 4, 2, 3>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
    if (mid >= 128) return launch_ring<2, 2, 2, 2, 4>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
    return launch_ring<2, 2, 1, 1, 4>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
  }
  // any K that is a multiple of 32: register-staged double buffer
  if (big >= 256) return launch<4, 4>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
  return launch<2, 2>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
}

// ---------------------------------------------------------------------------
// NVFP4 operands.  The scaled matrix core takes E8M0 scales per 32 elements only, and folding an
// E4M3 block scale into the elements would need q * V at up to 6 significant bits, more than any
// 8-bit float holds.  The exact route: decode each element to q * V (the block scale, without the
// tensor's global scale), which bfloat16 represents exactly (E2M1 has 2 significant bits, E4M3 4,
// and |q * V| lies in [2^-10, 2688]); multiply on the bf16 matrix cores (bf16 products are exact
// in the float32 accumulator); scale the result by fp32(S_a * S_b).

// E4M3 byte -> float (sign bit 7; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal)
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = (e == 0) ? (float)m * 0x1p-9f : (float)(8u + m) * __builtin_ldexpf(1.0f, (int)e - 10);
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return (b & 0x80u) ? -v : v;
}

// One lane per 16-element block: 8 code bytes + 1 scale byte -> 16 bfloat16 values (32 bytes).
// Blocks past K (up to kp, a multiple of 32) are written as zeros.  When a row holds a multiple of
// 64 blocks, a wave's output is one contiguous 2 KB run, stored in 1 KB pieces through LDS.
__global__ __launch_bounds__(256) void nvfp4_to_bf16_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales, int rows, int k,
                                                            int kp, uint16_t *__restrict__ out) {
  const int bpr = kp / 16;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)blockIdx.x * 256 + 64 * fp4q::wave_index();
  int r, blk;
  const bool valid = fp4q::lane_chunk(t0, lane, bpr, (int64_t)rows * bpr, r, blk);
  const bool whole = (bpr & 63) == 0;  // then every lane of a wave is valid or none is
  if (!valid) return;
  uint32_t w[8];
  if (blk * 16 < k) {
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + (int64_t)r * (k / 2) + blk * 8);
    const float V = e4m3_decode(scales[(int64_t)r * (k / 16) + blk]);
    // decode the 16 codes in element order: element 2i is the low nibble of byte i
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = i < 4 ? c.x : c.y;
      float2v q;
      switch (i & 3) {
        case 0: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
        case 1: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
        case 2: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
        default: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
      }
      // q * V is exact in float32 and in bfloat16, so dropping the low 16 bits is exact
      const uint32_t lo = __float_as_uint(q[0] * V) >> 16, hi = __float_as_uint(q[1] * V) >> 16;
      w[i] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0;
  }
  const fp4q::u32x4 q[2] = {fp4q::u32x4{w[0], w[1], w[2], w[3]}, fp4q::u32x4{w[4], w[5], w[6], w[7]}};
  fp4q::u32x4 *row = reinterpret_cast<fp4q::u32x4 *>(out + (int64_t)r * kp);
  if (whole) {
    __shared__ fp4q::WaveStage<2> stage[4];
    fp4q::wave_store<2>(row + 2 * (blk - lane), q, lane, stage[threadIdx.x >> 6]);
  } else {
    row[2 * blk] = q[0];
    row[2 * blk + 1] = q[1];
  }
}

// NVFP4 operands through the direct-to-LDS ring, decoded in registers (K a multiple of 128).  A stage
// is 128 K elements of every row: 64 code bytes (four 16-byte chunks, swizzled as in the MXFP4 ring)
// and 8 E4M3 scale bytes.  Lane half h of a wave owns elements 64 h .. 64 h + 63 of the stage (chunks
// 2 h and 2 h + 1, scale bytes 4 h .. 4 h + 3); k step ks (0 .. 7) feeds v_mfma_f32_32x32x16_f16
// with elements 64 h + 8 ks .. + 7 of every lane, in both operands alike, decoded to q * E4M3(p) in
// float16 (exact, as in the few-token kernel).  Steps run in ascending order within a stage, stages
// in ascending order; the accumulator is scaled by fp32(S_a S_b) at the end.  Staging FP4 codes
// instead of decoded bfloat16 cuts the LDS bytes per MFMA by four (the bfloat16 ring is bound by
// them), at the price of about one VALU instruction per element read.
template <int WGM, int WGN, int TM, int TN, int NS, typename OutT>
__global__ __launch_bounds__(64 * WGM * WGN) void nv_gemm_ring_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, int M, int N, int nst, int64_t kb, int64_t sbytes, const float *__restrict__ ga,
    const float *__restrict__ gb, OutT *__restrict__ C, int64_t ldc) {
  constexpr int WAVES = WGM * WGN;
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int ROWB = 64, SPR = 8;  // code and scale bytes per row per stage
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int SA_OFF = A_BYTES + B_BYTES, SB_OFF = SA_OFF + BM * SPR;
  constexpr int STAGE = SB_OFF + BN * SPR;
  constexpr int RPL = 1024 / ROWB;  // rows per 1 KB code load
  constexpr int A_INSTR = BM / RPL / WAVES, B_INSTR = BN / RPL / WAVES;
  constexpr int SA_INSTR = BM * SPR / 256, SB_INSTR = BN * SPR / 256;  // 256 B scale loads (32 rows)
  constexpr int SQ = (SA_INSTR + SB_INSTR + WAVES - 1) / WAVES;
  static_assert(A_INSTR * WAVES * RPL == BM && B_INSTR * WAVES * RPL == BN, "code loads must divide evenly");
  static_assert(SA_INSTR * 256 == BM * SPR && SB_INSTR * 256 == BN * SPR, "scale loads cover whole rows");
  constexpr int LOADS = A_INSTR + B_INSTR + SQ;  // per wave per stage
  constexpr int SPARE = NS * STAGE;               // target of the filler scale loads
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE + 256];
  __shared__ uint2 parts_tab[256];  // E4M3 byte -> (2^e, two float16 copies of m)
  const float alpha = (*ga) * (*gb);

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int l32 = lane & 31, h = lane >> 5;
  for (int i = tid; i < 256; i += 64 * WAVES) parts_tab[i] = nv_scale_parts((uint32_t)i);

  const uint8_t *srcA[A_INSTR];
  const uint8_t *srcB[B_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int row = (wave * A_INSTR + i) * RPL + lane / 4;
    srcA[i] = A + (int64_t)min(m0 + row, M - 1) * kb + 16 * ((lane % 4) ^ swz<ROWB>(row));
  }
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    const int row = (wave * B_INSTR + i) * RPL + lane / 4;
    srcB[i] = B + (int64_t)min(n0 + row, N - 1) * kb + 16 * ((lane % 4) ^ swz<ROWB>(row));
  }
  // scale load q: 32 rows, lane l loading dword l % 2 of row l / 2 (rows past M or N repeat the last)
  const uint8_t *srcS[SQ];
  int dstS[SQ];
#pragma unroll
  for (int j = 0; j < SQ; ++j) {
    const int q = wave + WAVES * j;
    const int rl = lane / 2, dw = lane % 2;
    if (q < SA_INSTR) {
      srcS[j] = As + (int64_t)min(m0 + 32 * q + rl, M - 1) * sbytes + 4 * dw;
      dstS[j] = SA_OFF + 256 * q;
    } else if (q < SA_INSTR + SB_INSTR) {
      const int qb = q - SA_INSTR;
      srcS[j] = Bs + (int64_t)min(n0 + 32 * qb + rl, N - 1) * sbytes + 4 * dw;
      dstS[j] = SB_OFF + 256 * qb;
    } else {
      srcS[j] = As + (int64_t)min(m0 + rl, M - 1) * sbytes + 4 * dw;
      dstS[j] = -1;
    }
  }
  auto issue = [&](int st, int slot) {
    uint8_t *base = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) load_lds16(srcA[i] + st * ROWB, base + (wave * A_INSTR + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i)
      load_lds16(srcB[i] + st * ROWB, base + A_BYTES + (wave * B_INSTR + i) * 1024);
#pragma unroll
    for (int j = 0; j < SQ; ++j) load_lds4(srcS[j] + st * SPR, dstS[j] >= 0 ? base + dstS[j] : smem + SPARE);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{0};

  auto stage_barrier = [&]() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

#pragma unroll
  for (int s = 0; s < NS; ++s) issue(min(s, nst - 1), s);
  wait_lgkmcnt0();  // this wave's parts_tab stores are complete ...
  wait_vmcnt<(NS - 1) * LOADS>();
  stage_barrier();  // ... and visible to every wave after the barrier

  int slot = 0;
  for (int st = 0; st < nst; ++st) {
    const uint8_t *base = smem + slot * STAGE;
    // this wave's operands of the stage: two 16-byte chunks and one scale dword per row block
    i32x4 ca[TM][2], cb[TN][2];
    uint32_t sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * TM * 32 + i * 32 + l32;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        ca[i][c] = *reinterpret_cast<const i32x4 *>(base + r * ROWB + 16 * ((2 * h + c) ^ swz<ROWB>(r)));
      sa[i] = *reinterpret_cast<const uint32_t *>(base + SA_OFF + SPR * r + 4 * h);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * TN * 32 + j * 32 + l32;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        cb[j][c] = *reinterpret_cast<const i32x4 *>(base + A_BYTES + r * ROWB + 16 * ((2 * h + c) ^ swz<ROWB>(r)));
      sb[j] = *reinterpret_cast<const uint32_t *>(base + SB_OFF + SPR * r + 4 * h);
    }
    // software pipeline: step ks + 1 is decoded while step ks's MFMAs run, one MFMA between every
    // six VALU instructions; steps 2 kp and 2 kp + 1 share a block, so a block's scale parts are
    // looked up every other step
    uint2 pa[TM], pb[TN];
    f16x8 av[TM], bv[TN];
    auto lookup = [&](int kp) {
#pragma unroll
      for (int i = 0; i < TM; ++i) pa[i] = parts_tab[(sa[i] >> (8 * kp)) & 0xFFu];
#pragma unroll
      for (int j = 0; j < TN; ++j) pb[j] = parts_tab[(sb[j] >> (8 * kp)) & 0xFFu];
    };
    auto decode = [&](int ks, f16x8 *a_out, f16x8 *b_out) {
#pragma unroll
      for (int i = 0; i < TM; ++i) a_out[i] = nv_decode8((uint32_t)ca[i][ks >> 2][ks & 3], pa[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) b_out[j] = nv_decode8((uint32_t)cb[j][ks >> 2][ks & 3], pb[j]);
    };
    lookup(0);
    decode(0, av, bv);
    unroll(std::make_integer_sequence<int, 8>{}, [&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      f16x8 an[TM], bn[TN];
      if constexpr (ks + 1 < 8) {
        if constexpr ((ks + 1) % 2 == 0) lookup((ks + 1) / 2);
        decode(ks + 1, an, bn);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      unroll(std::make_integer_sequence<int, TM * TN>{}, [&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
      });
      if constexpr (ks + 1 < 8) {
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = bn[j];
      }
    });
    __builtin_amdgcn_sched_barrier(0);
    const int next = slot == NS - 1 ? 0 : slot + 1;
    wait_lgkmcnt0();                 // this wave's reads of stage st are complete
    wait_vmcnt<(NS - 2) * LOADS>();  // stage st + 1 has landed
    stage_barrier();                 // ... for every wave, and nobody reads stage st any more
    issue(min(st + NS, nst - 1), slot);
    slot = next;
  }

  // epilogue through LDS, as in the MXFP4 ring
  __syncthreads();
  constexpr int WCOLS = TN * 32;
  constexpr int EPAD = 16 / (int)sizeof(OutT);
  constexpr int EROW = WCOLS + EPAD;
  constexpr int VEC = 16 / (int)sizeof(OutT);
  constexpr int LPR = WCOLS / VEC;
  constexpr int RPI = 64 / LPR;
  static_assert(WAVES * 32 * EROW * (int)sizeof(OutT) <= NS * STAGE, "epilogue staging must fit in the ring");
  OutT *stage_out = reinterpret_cast<OutT *>(smem) + wave * 32 * EROW;
  const int col0 = n0 + wn * WCOLS;
  const bool vec_ok = ((uintptr_t)C % 16 == 0) && ((ldc * (int64_t)sizeof(OutT)) % 16 == 0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        // registers v and v + 1 hold rows r and r + 1 of the same column
        const int r = 8 * (v >> 2) + 4 * h + (v & 3);
        OutT *o = stage_out + r * EROW + j * 32 + l32;
        if constexpr (sizeof(OutT) == 4) {
          o[0] = alpha * acc[i][j][v];
          o[EROW] = alpha * acc[i][j][v + 1];
        } else {
          const uint32_t p = f32x2_to_bf16x2(alpha * acc[i][j][v], alpha * acc[i][j][v + 1]);
          o[0] = (uint16_t)p;
          o[EROW] = (uint16_t)(p >> 16);
        }
      }
    const int row0 = m0 + wm * TM * 32 + i * 32;
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const int r = q * RPI + lane / LPR, c = (lane % LPR) * VEC;
      const int row = row0 + r, col = col0 + c;
      const i32x4 v = *reinterpret_cast<const i32x4 *>(stage_out + r * EROW + c);
      if (row < M) {
        OutT *dst = C + (int64_t)row * ldc + col;
        if (vec_ok && col + VEC <= N) {
          *reinterpret_cast<i32x4 *>(dst) = v;
        } else {
          const OutT *e = reinterpret_cast<const OutT *>(&v);
#pragma unroll
          for (int t = 0; t < VEC; ++t)
            if (col + t < N) dst[t] = e[t];
        }
      }
    }
  }
}

template <int WGM, int WGN, int TM, int TN, int NS, typename OutT>
hipError_t launch_nv_ring(const uint8_t *a, const uint8_t *as, const float *ga, const uint8_t *b, const uint8_t *bs,
                          const float *gb, int m, int n, int k, OutT *c, int64_t ldc, hipStream_t s) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  hipLaunchKernelGGL((nv_gemm_ring_kernel<WGM, WGN, TM, TN, NS, OutT>), dim3((unsigned)tiles), dim3(64 * WGM * WGN),
                     0, s, a, as, b, bs, m, n, k / 128, (int64_t)(k / 2), (int64_t)(k / 16), ga, gb, c, ldc);
  return hipGetLastError();
}

// NVFP4 operands decoded in registers (K a multiple of 128), for products too small for 256 x 256
// tiles on every CU: 128 x 128 or 64 x 64 tiles.  (With 256 x 256 tiles the decode, four waves'
// worth per A row and two per B row, outweighs the saved LDS traffic: the decode pass and the
// bfloat16 ring measured faster there.)
bool nv_ring_applies(int64_t m, int64_t n, int64_t k) {
  return k % 128 == 0 && ((m + 255) / 256) * ((n + 255) / 256) < 256;
}

template <typename OutT>
hipError_t dispatch_nv_ring(const uint8_t *a, const uint8_t *as, const float *ga, const uint8_t *b, const uint8_t *bs,
                            const float *gb, int m, int n, int k, OutT *c, int64_t ldc, hipStream_t s) {
  const int64_t mid = (int64_t)((m + 127) / 128) * ((n + 127) / 128);
  if (mid >= 128) return launch_nv_ring<2, 2, 2, 2, 4, OutT>(a, as, ga, b, bs, gb, m, n, k, c, ldc, s);
  return launch_nv_ring<2, 2, 1, 1, 4, OutT>(a, as, ga, b, bs, gb, m, n, k, c, ldc, s);
}

template <typename OutT>
hipError_t dispatch_nv(const uint16_t *a, const uint16_t *b, int m, int n, int kp, const float *ga, const float *gb,
                       OutT *c, int64_t ldc, hipStream_t s) {
  const int64_t big = (int64_t)((m + 255) / 256) * ((n + 255) / 256);
  const int64_t mid = (int64_t)((m + 127) / 128) * ((n + 127) / 128);
  // 128-byte stages pay off with the large tiles only (measured)
  if (big >= 256 && kp % 64 == 0)
    return launch_ring_bf16<2, 4, 4, 2, 2, OutT, 128>(a, b, m, n, kp, ga, gb, c, ldc, s);
  if (big >= 256) return launch_ring_bf16<2, 4, 4, 2, 3>(a, b, m, n, kp, ga, gb, c, ldc, s);
  if (mid >= 128) return launch_ring_bf16<2, 2, 2, 2, 4>(a, b, m, n, kp, ga, gb, c, ldc, s);
  return launch_ring_bf16<2, 2, 1, 1, 4>(a, b, m, n, kp, ga, gb, c, ldc, s);
}

int64_t padded_k(int64_t k) { return (k + 31) / 32 * 32; }

}  // namespace fp4q_gemm

extern "C" size_t fp4q_gemm_mxfp4_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0 || k % 32) return 0;
  return (size_t)fp4q_gemm::gemm_mxfp4_workspace(m, n, k);
}

extern "C" fp4q_status_t fp4q_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                                         const uint8_t *b_scales, int64_t m, int64_t n, int64_t k, float alpha,
                                         fp4q_dtype_t out_dtype, void *c, int64_t ldc, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  using namespace fp4q_gemm;
  if (out_dtype != FP4Q_F32 && out_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (m < 0 || n < 0 || k <= 0 || k % 32 || ldc < n) return FP4Q_ERR_SHAPE;
  if (m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31) || k >= ((int64_t)1 << 31)) return FP4Q_ERR_SHAPE;
  if (m == 0 || n == 0) return FP4Q_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4Q_ERR_NULL;
  const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
  if (tiles >= ((int64_t)1 << 31)) return FP4Q_ERR_SHAPE;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(c, out_dtype == FP4Q_F32 ? 4 : 2))
    return FP4Q_ERR_ALIGN;
  // the workspace is optional: with it (and K a multiple of 256) large products reorganise the scales
  // and few-token products split K
  uint8_t *ws = nullptr;
  const int64_t need = gemm_mxfp4_workspace(m, n, k);
  if (workspace && need > 0) {
    if (workspace_bytes < (size_t)need) return FP4Q_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP4Q_ERR_ALIGN;
    ws = (uint8_t *)workspace;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (out_dtype == FP4Q_F32)
    e = dispatch<float>(a_codes, a_scales, b_codes, b_scales, (int)m, (int)n, (int)k, alpha, (float *)c, ldc, s, ws);
  else
    e = dispatch<uint16_t>(a_codes, a_scales, b_codes, b_scales, (int)m, (int)n, (int)k, alpha, (uint16_t *)c, ldc,
                           s, ws);
  return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
}

extern "C" size_t fp4q_gemm_nvfp4_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0) return 0;
  // the few-token kernel decodes in registers; it needs room only for its K segments' partial sums
  const fp4q_gemm::NvSkinnyPlan plan = fp4q_gemm::nv_skinny_plan(m, n, k);
  if (plan.S) return plan.KS > 1 ? (size_t)(plan.KS * m * n * 4) : 0;
  return (size_t)((m + n) * fp4q_gemm::padded_k(k) * 2);
}

extern "C" fp4q_status_t fp4q_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_global,
                                         const uint8_t *b_codes, const uint8_t *b_scales, const float *b_global,
                                         int64_t m, int64_t n, int64_t k, fp4q_dtype_t out_dtype, void *c,
                                         int64_t ldc, void *workspace, size_t workspace_bytes, void *stream) {
  using namespace fp4q_gemm;
  if (out_dtype != FP4Q_F32 && out_dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (m < 0 || n < 0 || k <= 0 || k % 16 || ldc < n) return FP4Q_ERR_SHAPE;
  if (m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31) || k >= ((int64_t)1 << 30)) return FP4Q_ERR_SHAPE;
  if (m == 0 || n == 0) return FP4Q_OK;
  if (!a_codes || !a_scales || !a_global || !b_codes || !b_scales || !b_global || !c) return FP4Q_ERR_NULL;
  const int64_t kp = padded_k(k);
  if (((m + 127) / 128) * ((n + 127) / 128) >= ((int64_t)1 << 31) || (m + n) * (kp / 16) >= ((int64_t)1 << 40))
    return FP4Q_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  // few tokens: the few-token kernel decodes both operands in registers (a workspace only for the
  // partial sums of its K segments)
  const NvSkinnyPlan plan = nv_skinny_plan(m, n, k);
  if (plan.S) {
    if (plan.KS > 1 && (!workspace || workspace_bytes < fp4q_gemm_nvfp4_workspace_bytes(m, n, k)))
      return FP4Q_ERR_WORKSPACE;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 16) || !aligned(b_scales, 16) ||
        !aligned(a_global, 4) || !aligned(b_global, 4) || !aligned(c, out_dtype == FP4Q_F32 ? 4 : 2) ||
        (plan.KS > 1 && !aligned(workspace, 16)))
      return FP4Q_ERR_ALIGN;
    float *parts = plan.KS > 1 ? (float *)workspace : nullptr;
    const hipError_t e =
        out_dtype == FP4Q_F32
            ? launch_nv_skinny<float>(a_codes, a_scales, a_global, b_codes, b_scales, b_global, (int)m, (int)n,
                                      (int)k, plan, (float *)c, ldc, parts, s)
            : launch_nv_skinny<uint16_t>(a_codes, a_scales, a_global, b_codes, b_scales, b_global, (int)m, (int)n,
                                         (int)k, plan, (uint16_t *)c, ldc, parts, s);
    return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
  }
  if (!workspace || workspace_bytes < fp4q_gemm_nvfp4_workspace_bytes(m, n, k)) return FP4Q_ERR_WORKSPACE;
  if (!aligned(a_codes, 8) || !aligned(b_codes, 8) || !aligned(a_global, 4) || !aligned(b_global, 4) ||
      !aligned(workspace, 16) || !aligned(c, out_dtype == FP4Q_F32 ? 4 : 2))
    return FP4Q_ERR_ALIGN;
  if (nv_ring_applies(m, n, k) && aligned(a_codes, 16) && aligned(b_codes, 16) && aligned(a_scales, 4) &&
      aligned(b_scales, 4)) {
    // codes staged in LDS and decoded in registers (the workspace is not touched)
    const hipError_t e =
        out_dtype == FP4Q_F32
            ? dispatch_nv_ring<float>(a_codes, a_scales, a_global, b_codes, b_scales, b_global, (int)m, (int)n,
                                      (int)k, (float *)c, ldc, s)
            : dispatch_nv_ring<uint16_t>(a_codes, a_scales, a_global, b_codes, b_scales, b_global, (int)m, (int)n,
                                         (int)k, (uint16_t *)c, ldc, s);
    return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
  }
  uint16_t *wa = (uint16_t *)workspace;
  uint16_t *wb = wa + m * kp;
  const int64_t ta = m * (kp / 16), tb = n * (kp / 16);
  hipLaunchKernelGGL(nvfp4_to_bf16_kernel, dim3((unsigned)((ta + 255) / 256)), dim3(256), 0, s, a_codes, a_scales,
                     (int)m, (int)k, (int)kp, wa);
  hipLaunchKernelGGL(nvfp4_to_bf16_kernel, dim3((unsigned)((tb + 255) / 256)), dim3(256), 0, s, b_codes, b_scales,
                     (int)n, (int)k, (int)kp, wb);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    if (out_dtype == FP4Q_F32)
      e = dispatch_nv<float>(wa, wb, (int)m, (int)n, (int)kp, a_global, b_global, (float *)c, ldc, s);
    else
      e = dispatch_nv<uint16_t>(wa, wb, (int)m, (int)n, (int)kp, a_global, b_global, (uint16_t *)c, ldc, s);
  }
  return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
}
