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
// A workgroup of four waves (2 x 2) computes a BM x BN tile of C.  Each
// wave computes TM x TN blocks of 32 x 32, with the accumulators in
// registers.  K advances in stages of 128 elements: 64 bytes of codes and 4
// scale bytes per row of A and B.  A stage is loaded from global memory
// into registers while the matrix cores consume the previous stage from
// LDS (double buffer, one barrier per stage).  LDS rows are padded from 64
// to 80 bytes, so a wave's 16-byte operand reads hit distinct banks.
// Workgroups are renumbered so that each XCD (dispatched round-robin) gets
// a contiguous range of tiles, taken in groups of tile rows, and tiles that
// share A or B panels share an L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_gemm.h"

namespace fp4q_gemm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kKc = 128;     // K elements per stage
constexpr int kLdsRow = 80;  // bytes per staged row (64 + 16 padding)
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;  // tile rows per group in the tile order

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);  // quiet NaN
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

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

template <typename OutT>
hipError_t dispatch(const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs, int m, int n, int k,
                    float alpha, OutT *c, int64_t ldc, hipStream_t s) {
  // 256 x 256 tiles when they fill the chip at least once, else 128 x 128
  const int64_t big = (int64_t)((m + 255) / 256) * ((n + 255) / 256);
  if (big >= 256) return launch<4, 4>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
  return launch<2, 2>(a, as, b, bs, m, n, k, alpha, c, ldc, s);
}

}  // namespace fp4q_gemm

extern "C" fp4q_status_t fp4q_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                                         const uint8_t *b_scales, int64_t m, int64_t n, int64_t k, float alpha,
                                         fp4q_dtype_t out_dtype, void *c, int64_t ldc, void *stream) {
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
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (out_dtype == FP4Q_F32)
    e = dispatch<float>(a_codes, a_scales, b_codes, b_scales, (int)m, (int)n, (int)k, alpha, (float *)c, ldc, s);
  else
    e = dispatch<uint16_t>(a_codes, a_scales, b_codes, b_scales, (int)m, (int)n, (int)k, alpha, (uint16_t *)c, ldc,
                           s);
  return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
}
