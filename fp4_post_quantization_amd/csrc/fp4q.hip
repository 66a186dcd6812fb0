// fp4q: FP4 microscaling block quantization with block-scale search for
// gfx950 (MI355X).  Kernels and the C ABI declared in include/fp4q.h.
//
// Work decomposition (all kernels): a lane owns 16 contiguous elements of a
// row ("chunk"); an NVFP4 block is one lane, an MXFP4 block two adjacent
// lanes, an n-point Hadamard group n/16 adjacent lanes.  Block losses are
// accumulated inside the lane (plus one DPP exchange for MXFP4), so the
// candidate sweep needs no LDS traffic for data and no barriers.
//
// The quantize kernels map a wave to a tile of 64 consecutive chunks of a
// column band times a few rows; the per-column importance of WMSE is loaded
// into registers once per tile and reused for every row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <stdlib.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "fp4q.h"
#include "fp4q_device.h"

namespace fp4q {

// ============================================================ tables =====

// Values and correctly rounded reciprocals of the non-negative E4M3 patterns
// (index = pattern; entries 0 and 127 are 1.0), evaluated at compile time.
struct E4M3Tables {
  float v[128];
  float r[128];
};

constexpr float e4m3_value_const(int p) {
  float scale = 1.0f;  // 2^(exponent - 7)
  const int ef = p >> 3;
  if (ef == 0) return (float)p * 0.001953125f;  // subnormal p * 2^-9
  for (int k = 7; k > ef; --k) scale *= 0.5f;
  for (int k = 7; k < ef; ++k) scale *= 2.0f;
  return (1.0f + (float)(p & 7) * 0.125f) * scale;
}

constexpr E4M3Tables make_e4m3_tables() {
  E4M3Tables t{};
  for (int p = 0; p < 128; ++p) {
    const float v = (p >= 1 && p <= 126) ? e4m3_value_const(p) : 1.0f;
    t.v[p] = v;
    t.r[p] = 1.0f / v;  // IEEE division, correctly rounded
  }
  return t;
}

__constant__ E4M3Tables kE4M3 = make_e4m3_tables();

// ============================================================ kernels ====

// Global scale of an empty NVFP4 tensor (max over nothing = 0).
__global__ void zero_scale_kernel(float *global_scale) { *global_scale = 0.0f; }

// Where the global-max pass puts its results.
struct AmaxOut {
  uint32_t *partials;  // [gridDim.x] per-workgroup maxima
  uint32_t *status;
  const float *imp;    // importance [imp_n] to validate, or null
  int imp_n;
};

// End of a global-max pass: m is this thread's maximum |bits|; the
// workgroup's maximum goes to partials[blockIdx.x].  The workgroups also
// validate the importance vector between them (a strided slice each), so
// the quantizer that follows need not.
__device__ void finish_amax(uint32_t m, const AmaxOut &o) {
  __shared__ uint32_t red[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (o.imp) {
    bool ok = true;
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < o.imp_n; i += gridDim.x * kThreads)
      ok &= (o.imp[i] >= 0.0f) & (o.imp[i] <= 3.402823466e38f);
    if (!ok) atomicOr(o.status, FP4Q_DATA_BAD_IMPORTANCE);
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = red[k] > r ? red[k] : r;
    o.partials[blockIdx.x] = r;
  }
}

// Per-workgroup maximum of |x| (after the optional rotation) as a float32
// bit pattern.  Integer order of |bits| is float order for finite values,
// and any Inf/NaN yields a pattern >= 0x7F800000.
template <typename T, int HAD>
__global__ __launch_bounds__(kThreads) void amax_kernel(const T *__restrict__ x, int64_t ld, int cpr,
                                                         int total, AmaxOut o) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
  const int stride = gridDim.x * kThreads;
  for (int g = blockIdx.x * kThreads + threadIdx.x; g < total; g += stride) {
    const int r = g / cpr, c = g - r * cpr;
    float z[16];
    load16(x + (int64_t)r * ld + (int64_t)c * 16, z);
    if constexpr (HAD != 0) fwht<HAD>(z, lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = as_u(z[i]) & 0x7FFFFFFFu;
      m = b > m ? b : m;
    }
  }
  finish_amax(m, o);
}

// Same maximum for a contiguous, unrotated matrix viewed as n_vec 16-byte
// vectors; eight independent loads per thread are in flight per iteration.
template <typename T>
__device__ __forceinline__ uint32_t fold_abs_bits(uint32_t m, u32x4 v) {
  if constexpr (sizeof(T) == 2) {  // two bf16 per dword
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = v[k] & 0x7FFFu, hi = (v[k] >> 16) & 0x7FFFu;
      m = max(m, max(lo, hi));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, v[k] & 0x7FFFFFFFu);
  }
  return m;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const u32x4 *__restrict__ v, int64_t n_vec,
                                                              AmaxOut o) {
  constexpr int U = 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  for (; i + (U - 1) * stride < n_vec; i += U * stride) {
    u32x4 a[U];
#pragma unroll
    for (int k = 0; k < U; ++k) a[k] = v[i + k * stride];
#pragma unroll
    for (int k = 0; k < U; ++k) m = fold_abs_bits<T>(m, a[k]);
  }
  for (; i < n_vec; i += stride) m = fold_abs_bits<T>(m, v[i]);
  if constexpr (sizeof(T) == 2) m <<= 16;  // bf16 pattern -> float32 pattern
  finish_amax(m, o);
}

// Maximum of |rotated x| for a contiguous matrix viewed as total chunks of
// 16 elements: Hadamard groups never straddle rows (cols is a multiple of
// n), so consecutive chunks form the groups whatever the row length.  Four
// chunks per thread are loaded before any is used.  stride is a multiple of
// 64 and total of HAD/16, so the lanes of a group enter and leave every
// branch together.
template <typename T, int HAD>
__global__ __launch_bounds__(kThreads) void amax_chunks_kernel(const T *__restrict__ x, int64_t total,
                                                                AmaxOut o) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  for (; g + (U - 1) * stride < total; g += U * stride) {
    Raw<T> r[U];
#pragma unroll
    for (int k = 0; k < U; ++k) load_raw(x + (g + k * stride) * 16, r[k]);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float z[16];
      widen(r[k], z);
      fwht<HAD>(z, lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = max(m, as_u(z[i]) & 0x7FFFFFFFu);
    }
  }
  for (; g < total; g += stride) {
    Raw<T> r;
    load_raw(x + g * 16, r);
    float z[16];
    widen(r, z);
    fwht<HAD>(z, lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, as_u(z[i]) & 0x7FFFFFFFu);
  }
  finish_amax(m, o);
}

struct SweepArgs {
  const void *x;
  int64_t ld;
  int rows, cols, cpr;          // cpr = chunks (16 columns) per row
  const float *imp;             // [cols] or null
  int off_lo, off_hi;
  int rows_per_tile, nbands, ntiles;
  const uint32_t *partials;     // amax partials (NVFP4, computed scale)
  int n_partials;
  bool check_imp;               // validate the importance (no global-max pass did)
  const float *given_scale;     // NVFP4 with FP4Q_GIVEN_SCALE, else null
  uint8_t *codes, *scales;
  float *gscale_out;            // NVFP4 global scale output (computed scale)
  float *loss;
  int8_t *offs;
  uint32_t *status;
};

__device__ __forceinline__ void load_importance(const float *p, float w[16]) {
  const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 v = q[k];
    w[4 * k] = v.x;
    w[4 * k + 1] = v.y;
    w[4 * k + 2] = v.z;
    w[4 * k + 3] = v.w;
  }
}

__device__ __forceinline__ bool importance_ok(const float w[16]) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 16; ++i) ok &= (w[i] >= 0.0f) & (w[i] <= 3.402823466e38f);
  return ok;
}

// Codes of 8 values, optionally halved first: the scale operand 2.0 makes
// the hardware convert y / 2 (exactly, checked on every float32 below 2^21).
// All four bytes of the result are written, so `old` only carries a register.
template <bool HALF>
__device__ __forceinline__ uint32_t cvt8(const float y[8], uint32_t old) {
  const float sc = HALF ? 2.0f : 1.0f;
  old = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[0], y[1], sc, 0);
  old = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[2], y[3], sc, 1);
  old = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[4], y[5], sc, 2);
  old = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y[6], y[7], sc, 3);
  return old;
}

// Loss of one candidate over this lane's 16 elements from their codes:
// e_i = fp32(us_i - q_i*V), summed in element order with one rounding per
// term, acc <- fma(t_i, e_i, acc), t_i = e_i (MSE) or fp32(w_i * e_i) (WMSE).
// us and q carry the sign of x (the conversions are sign-symmetric), so e_i
// is the error up to its sign and t_i * e_i is unchanged; q*V is exact, so
// fmaf(-q, V, us) is exactly fp32(us - q*V).
template <bool WMSE>
__device__ __forceinline__ float loss_of_codes(const float us[16], const float w[16], uint32_t pk0,
                                               uint32_t pk1, float V) {
  float q[16];
  fp4x8_to_f32(pk0, q);
  fp4x8_to_f32(pk1, q + 8);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = fmaf(-q[i], V, us[i]);
    acc = fmaf(WMSE ? w[i] * e : e, e, acc);
  }
  return acc;
}

// Keep the candidate with the least loss; among equal losses the smallest
// pattern / exponent, whatever order the candidates are visited in.
__device__ __forceinline__ bool consider(float L, int p, bool ok, float &Lbest, int &pbest) {
  const bool take = ok & ((L < Lbest) | ((L == Lbest) & (p < pbest)));
  Lbest = take ? L : Lbest;
  pbest = take ? p : pbest;
  return take;
}

// ScaleSweep candidate search for one block (this lane's 16 elements).
// Offsets pair up octet by octet, [lo, lo+8) with [lo+8, lo+16), ...; the
// lower and the upper members are tracked as two running minima, each
// visited in ascending pattern order with a strict "<", and merged with the
// smallest-pattern tie rule.  CHECKED handles windows that leave the normal
// E4M3 range (clamping, validity, subnormal lower members).  Returns p*.
template <bool WMSE, bool CHECKED>
__device__ __forceinline__ int nv_sweep(const float us[16], const float w[16], int base, int lo, int hi,
                                        const float *Vtab, const float *Rtab, float &Lout) {
  const int plo = max(1, base + lo);
  float La = __builtin_inff(), Lb = __builtin_inff();
  int pa = plo, pb = 0x7FFFFFFF;
  uint32_t k0 = 0, k1 = 0, h0 = 0, h1 = 0;
  for (int o = lo; o <= hi; ++o) {
    if (((o - lo) >> 3) & 1) continue;  // visited as the upper member of a pair
    const int p = base + o;
    bool ok = true;
    int pc = p;
    if constexpr (CHECKED) {
      ok = (p >= 1) & (p <= 126);
      pc = min(max(p, 1), 126);
    }
    float y[16];
    const float R = Rtab[pc];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = us[i] * R;
    k0 = cvt8<false>(y, k0);
    k1 = cvt8<false>(y + 8, k1);
    if (o + 8 <= hi) {
      const int ph = p + 8;
      bool okh = true;
      int phc = ph;
      if constexpr (CHECKED) {
        okh = (ph >= 1) & (ph <= 126);
        phc = min(max(ph, 1), 126);
        if (p >= 8) {
          h0 = cvt8<true>(y, h0);
          h1 = cvt8<true>(y + 8, h1);
        } else {  // E4M3 subnormal lower member: no exact factor 2
          const float Rh = Rtab[phc];
          float y2[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) y2[i] = us[i] * Rh;
          h0 = cvt8<false>(y2, h0);
          h1 = cvt8<false>(y2 + 8, h1);
        }
      } else {
        h0 = cvt8<true>(y, h0);  // y / 2 == fp32(us * R[p + 8]) exactly
        h1 = cvt8<true>(y + 8, h1);
      }
      const float L = loss_of_codes<WMSE>(us, w, h0, h1, Vtab[phc]);
      const bool take = okh & (L < Lb);
      Lb = take ? L : Lb;
      pb = take ? ph : pb;
    }
    const float L = loss_of_codes<WMSE>(us, w, k0, k1, Vtab[pc]);
    const bool take = ok & (L < La);
    La = take ? L : La;
    pa = take ? p : pa;
  }
  const bool upper = (Lb < La) | ((Lb == La) & (pb < pa));
  Lout = upper ? Lb : La;
  return upper ? pb : pa;
}

// NVFP4 ScaleSweep: one lane per 16-element block.
//
// Candidates p and p + 8 (both >= 8) have E4M3 values V and 2V, so
// fp32(u * R[p+8]) = fp32(u * R[p]) / 2 exactly and the pair shares one set
// of products u * R; the upper member is converted with the halving scale.
template <typename T, bool WMSE, int HAD>
__global__ __launch_bounds__(kThreads) void nvfp4_sweep_kernel(SweepArgs a) {
  __shared__ float Vtab[128], Rtab[128];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();

  if (tid < 128) {
    Vtab[tid] = kE4M3.v[tid];
    Rtab[tid] = kE4M3.r[tid];
  }
  const int tile = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wave);
  const int band = tile % a.nbands, rg = tile / a.nbands;
  const int c = band * 64 + lane;
  const bool active = tile < a.ntiles && c < a.cpr;  // whole Hadamard groups are active or not together
  const int r0 = rg * a.rows_per_tile;
  const int r1 = min(a.rows, r0 + a.rows_per_tile);
  const T *xc = static_cast<const T *>(a.x) + (int64_t)c * 16;
  // the importance and the first row are loaded before S is known: their latency overlaps the
  // reduction below
  float w[16];
  Raw<T> cur, nxt;
  if (active) {
    if constexpr (WMSE) load_importance(a.imp + (int64_t)c * 16, w);
    load_raw(xc + (int64_t)r0 * a.ld, cur);
  }
  // wave 0 finds S and S_inv (the maximum of the global-max partials, or the given scale) for the
  // workgroup
  __shared__ float sc[2];
  if (wave == 0) {
    float S;
    if (a.given_scale) {
      S = *a.given_scale;
      if (blockIdx.x == 0 && lane == 0 && (!(S >= 0.0f) || isinf(S)))
        atomicOr(a.status, FP4Q_DATA_BAD_GLOBAL_SCALE);
    } else {
      uint32_t m = 0;
      for (int i = lane; i < a.n_partials; i += 64) m = max(m, a.partials[i]);
      m = wave_max_u32(m);
      S = as_f(m) / 1536.0f;  // max|x| / (256 * 6), correctly rounded
      if (blockIdx.x == 0 && lane == 0) {
        *a.gscale_out = S;
        if (m >= 0x7F800000u) atomicOr(a.status, FP4Q_DATA_NONFINITE_INPUT);
      }
    }
    if (lane == 0) {
      sc[0] = S;
      sc[1] = (S == 0.0f) ? 0.0f : 1.0f / S;
    }
  }
  __syncthreads();
  const float S = sc[0], S_inv = sc[1];
  const float SS = S * S;
  if (!active) return;
  if constexpr (WMSE) {
    if (a.check_imp && !importance_ok(w)) atomicOr(a.status, FP4Q_DATA_BAD_IMPORTANCE);
  }

  const int bpr = a.cpr;  // blocks per row
  const int lo = a.off_lo, hi = a.off_hi;
  for (int r = r0; r < r1; ++r) {
    if (r + 1 < r1) load_raw(xc + (int64_t)(r + 1) * a.ld, nxt);
    float z[16];
    widen(cur, z);
    if constexpr (HAD != 0) fwht<HAD>(z, lane);

    // signed magnitudes in units of S: |us| = fp32(|x| * S_inv) exactly
    float us[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      us[i] = z[i] * S_inv;
      amax = fmaxf(amax, fabsf(us[i]));
    }
    // with a computed scale the global-max pass already reported non-finite x
    if (a.given_scale) {
      bool finite = true;
#pragma unroll
      for (int i = 0; i < 16; ++i) finite &= fabsf(z[i]) <= 3.402823466e38f;
      if (!finite) atomicOr(a.status, FP4Q_DATA_NONFINITE_INPUT);
    }
    const float t = amax / 6.0f;  // correctly rounded
    int base = e4m3_rne_sat(t);
    base = base < 1 ? 1 : base;
    float Lbest;
    int pbest;
    // all candidates of every lane normal E4M3 patterns: no clamping, no
    // validity tests, every pair related by an exact factor 2
    const bool interior = (base + lo >= 8) & (base + hi <= 126);
    if (__all(interior))
      pbest = nv_sweep<WMSE, false>(us, w, base, lo, hi, Vtab, Rtab, Lbest);
    else
      pbest = nv_sweep<WMSE, true>(us, w, base, lo, hi, Vtab, Rtab, Lbest);

    const float Rb = Rtab[pbest];
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = us[i] * Rb;
    const uint32_t c0 = cvt8<false>(y, 0u), c1 = cvt8<false>(y + 8, 0u);
    *reinterpret_cast<uint2 *>(a.codes + (int64_t)r * (a.cols / 2) + (int64_t)c * 8) = make_uint2(c0, c1);
    const int64_t bi = (int64_t)r * bpr + c;
    a.scales[bi] = (uint8_t)pbest;
    if (a.loss) a.loss[bi] = Lbest * SS;
    if (a.offs) a.offs[bi] = (int8_t)(pbest - base);
    cur = nxt;
  }
}

// MXFP4 exponent sweep for one block (this lane's 16 elements and its
// partner lane's): exponents E and E + 1 pair up, E + 1 converted from the
// products of E with the halving scale.  Returns E*; Lbest gets its loss
// and, KEEP, b0 / b1 its codes.
template <bool WMSE, bool KEEP>
__device__ __forceinline__ int mx_sweep(const float z[16], const float w[16], int eb, int lo, int hi, float &Lbest,
                                        uint32_t &b0, uint32_t &b1) {
  Lbest = __builtin_inff();
  int ebest = max(-127, eb + lo);
  uint32_t k0 = 0, k1 = 0, h0 = 0, h1 = 0;
  for (int o = lo; o <= hi; o += 2) {
    const int E = eb + o;
    const bool ok = (E >= -127) & (E <= 127);
    const int Ec = min(max(E, -127), 127);
    const float down = pow2f(-Ec);
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = z[i] * down;
    k0 = cvt8<false>(y, k0);
    k1 = cvt8<false>(y + 8, k1);
    if (o + 1 <= hi) {
      const int E1 = E + 1;
      const bool ok1 = (E1 >= -127) & (E1 <= 127);
      const int E1c = min(max(E1, -127), 127);
      if (E >= -127) {
        h0 = cvt8<true>(y, h0);
        h1 = cvt8<true>(y + 8, h1);
      } else {  // lower member clamped: convert the upper one directly
        const float d1 = pow2f(-E1c);
        float y2[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y2[i] = z[i] * d1;
        h0 = cvt8<false>(y2, h0);
        h1 = cvt8<false>(y2 + 8, h1);
      }
      const float half1 = loss_of_codes<WMSE>(z, w, h0, h1, pow2f(E1c));
      const bool t1 = consider(half1 + xor_lane<1>(half1), E1, ok1, Lbest, ebest);
      if constexpr (KEEP) {
        b0 = t1 ? h0 : b0;
        b1 = t1 ? h1 : b1;
      }
    }
    const float half0 = loss_of_codes<WMSE>(z, w, k0, k1, pow2f(Ec));
    const bool t0 = consider(half0 + xor_lane<1>(half0), E, ok, Lbest, ebest);
    if constexpr (KEEP) {
      b0 = t0 ? k0 : b0;
      b1 = t0 ? k1 : b1;
    }
  }
  return ebest;
}

// MXFP4 exponent sweep: two adjacent lanes per 32-element block.  Exponents
// E and E + 1 form pairs: fp32(x * 2^-(E+1)) = fp32(x * 2^-E) / 2.
template <typename T, bool WMSE, int HAD>
__global__ __launch_bounds__(kThreads) void mxfp4_sweep_kernel(SweepArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int tile = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wave);
  if (tile >= a.ntiles) return;
  const int band = tile % a.nbands, rg = tile / a.nbands;
  const int c = band * 64 + lane;
  const bool active = c < a.cpr;  // cpr is even: both lanes of a block agree
  const int r0 = rg * a.rows_per_tile;
  const int r1 = min(a.rows, r0 + a.rows_per_tile);

  float w[16];
  if constexpr (WMSE) {
    if (active) {
      load_importance(a.imp + (int64_t)c * 16, w);
      if (a.check_imp && !importance_ok(w)) atomicOr(a.status, FP4Q_DATA_BAD_IMPORTANCE);
    }
  }
  if (!active) return;

  const T *xc = static_cast<const T *>(a.x) + (int64_t)c * 16;
  const int bpr = a.cpr / 2;
  const bool even = (lane & 1) == 0;
  const int lo = a.off_lo, hi = a.off_hi;
  // short windows keep the winner's codes (two selects per candidate) instead of converting again
  const bool keep = hi - lo < 8;
  Raw<T> cur, nxt;
  load_raw(xc + (int64_t)r0 * a.ld, cur);
  for (int r = r0; r < r1; ++r) {
    if (r + 1 < r1) load_raw(xc + (int64_t)(r + 1) * a.ld, nxt);
    float z[16];
    widen(cur, z);
    if constexpr (HAD != 0) fwht<HAD>(z, lane);

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(z[i]));
    amax = fmaxf(amax, xor_lane<1>(amax));
    const int eb = mx_base_exponent(amax);

    float Lbest;
    uint32_t b0 = 0, b1 = 0;  // codes of the best candidate (short windows)
    const int ebest = keep ? mx_sweep<WMSE, true>(z, w, eb, lo, hi, Lbest, b0, b1)
                           : mx_sweep<WMSE, false>(z, w, eb, lo, hi, Lbest, b0, b1);

    // A non-finite element makes its e, and so every candidate's loss, NaN or infinite (the terms
    // t * e are never negative), so a finite best loss proves the block finite; the elementwise
    // test runs only when it is not (an overflowing loss of finite data also lands there).
    const bool lfin = Lbest <= 3.402823466e38f;
    if (!lfin) {
      bool finite = true;
#pragma unroll
      for (int i = 0; i < 16; ++i) finite &= fabsf(z[i]) <= 3.402823466e38f;
      if (!finite) atomicOr(a.status, FP4Q_DATA_NONFINITE_INPUT);
    }
    uint32_t k0 = b0, k1 = b1;  // a finite best loss was taken, and its codes with it
    if (!(keep & lfin)) {
      const float db = pow2f(-ebest);
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = z[i] * db;
      k0 = cvt8<false>(y, 0u);
      k1 = cvt8<false>(y + 8, 0u);
    }
    *reinterpret_cast<uint2 *>(a.codes + (int64_t)r * (a.cols / 2) + (int64_t)c * 8) = make_uint2(k0, k1);
    if (even) {
      const int64_t bi = (int64_t)r * bpr + (c >> 1);
      a.scales[bi] = (uint8_t)(ebest + 127);
      if (a.loss) a.loss[bi] = Lbest;
      if (a.offs) a.offs[bi] = (int8_t)(ebest - eb);
    }
    cur = nxt;
  }
}

// 16 floats of chunk c of an output row (row stride 16 cpr floats).  When
// the row length is a multiple of 64 chunks, a wave's 64 chunks are one
// contiguous 4 KB run and go out as four 1 KB stores through LDS.
__device__ __forceinline__ void store_chunk_f32(float *row, int c, int cpr, int lane, const float v[16]) {
  u32x4 q[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = u32x4{as_u(v[4 * k]), as_u(v[4 * k + 1]), as_u(v[4 * k + 2]), as_u(v[4 * k + 3])};
  if ((cpr & 63) == 0) {
    __shared__ WaveStage<4> stage[kWaves];
    wave_store<4>(reinterpret_cast<u32x4 *>(row) + 4 * (c - lane), q, lane, stage[threadIdx.x >> 6]);
  } else {
    u32x4 *o = reinterpret_cast<u32x4 *>(row) + 4 * c;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = q[k];
  }
}

// FOCUS forward quantizer: one lane per 16-element chunk (flat over
// rows x chunks); the codes use the quantization scale Vc = V * c_k of each
// sub-block, the optional dequantized output the stored scale V alone.
template <typename T, int FMT, int SUB>
__global__ __launch_bounds__(kThreads) void relaxed_quant_kernel(const T *__restrict__ x, int64_t ld, int cpr,
                                                                  int cols, int total,
                                                                  const uint8_t *__restrict__ scales,
                                                                  const float *__restrict__ gscale,
                                                                  const uint16_t *__restrict__ coeffs,
                                                                  uint8_t *__restrict__ codes,
                                                                  float *__restrict__ dq,
                                                                  uint32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t g0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kThreads + (threadIdx.x & ~63u)));
  int r, c;
  if (!lane_chunk(g0, lane, cpr, total, r, c)) return;
  float z[16];
  load16(x + (int64_t)r * ld + (int64_t)c * 16, z);

  bool bad = false;
  float V, S_inv = 1.0f, S = 1.0f;
  if constexpr (FMT == FP4Q_NVFP4) {
    const int p = scales[(int64_t)r * cpr + c];
    bad |= (p < 1) | (p > 126);
    V = kE4M3.v[p & 127];
    S = *gscale;
    S_inv = (S == 0.0f) ? 0.0f : 1.0f / S;
  } else {
    const int b = scales[(int64_t)r * (cpr / 2) + (c >> 1)];
    bad |= b == 255;
    V = pow2f(min(b, 254) - 127);
  }
  bool finite = true;
  float us[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    finite &= fabsf(z[i]) <= 3.402823466e38f;
    us[i] = FMT == FP4Q_NVFP4 ? z[i] * S_inv : z[i];
  }
  // coefficients of this lane's sub-blocks: 16/SUB of them, or one shared
  // by the two lanes of a 32-element sub-block
  constexpr int NS = SUB >= 16 ? 1 : 16 / SUB;
  const int64_t crow = (int64_t)r * (cols / SUB);
  float y[16];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int64_t ci = SUB == 32 ? crow + (c >> 1) : crow + (int64_t)c * (16 / min(SUB, 16)) + j;
    const float cf = coeffs ? (float)__builtin_bit_cast(_Float16, coeffs[ci]) : 1.0f;
    bad |= !((cf > 0.0f) & (cf <= 65504.0f));
    const float R = 1.0f / (V * cf);
    bad |= !(R <= 3.402823466e38f);
    constexpr int E = SUB >= 16 ? 16 : SUB;
#pragma unroll
    for (int i = 0; i < E; ++i) y[j * E + i] = us[j * E + i] * R;
  }
  if (bad) atomicOr(status, FP4Q_DATA_BAD_SCALE);
  if (!finite) atomicOr(status, FP4Q_DATA_NONFINITE_INPUT);
  const uint32_t k0 = cvt8<false>(y, 0u), k1 = cvt8<false>(y + 8, 0u);
  *reinterpret_cast<uint2 *>(codes + (int64_t)r * (cols / 2) + (int64_t)c * 8) = make_uint2(k0, k1);
  if (dq) {
    float q[16];
    fp4x8_to_f32(k0, q);
    fp4x8_to_f32(k1, q + 8);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float m = q[i] * V;  // exact
      v[i] = FMT == FP4Q_NVFP4 ? m * S : m;
    }
    store_chunk_f32(dq + (int64_t)r * cols, c, cpr, lane, v);
  }
}

// ================================================================ GPTQ ====
// Column-by-column NVFP4 quantization with error feedback through the
// inverse-Hessian factor U (upper Cholesky factor of H^-1), in lazy
// batches of 128 columns; each 16-column group's scale comes from the
// ScaleSweep candidate search on the group's current values.

constexpr int kGptqBatch = 128;
// Columns past the current block of kGptqBlock receive the block's updates in one contraction.
constexpr int kGptqBlock = 1024;
static_assert(kGptqBlock % kGptqBatch == 0, "blocks hold whole batches");

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Global scale from the max-pass partials (a single workgroup).
__global__ __launch_bounds__(kThreads) void scale_from_partials_kernel(const uint32_t *__restrict__ partials,
                                                                        int n, float *__restrict__ gscale,
                                                                        uint32_t *__restrict__ status) {
  __shared__ uint32_t red[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) m = max(m, partials[i]);
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kWaves; ++i) m = max(m, red[i]);
    m = max(m, red[0]);
    *gscale = as_f(m) / 1536.0f;
    if (m >= 0x7F800000u) atomicOr(status, FP4Q_DATA_NONFINITE_INPUT);
  }
}


__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// One batch of 128 columns [i1, i1 + 128).  A row is handled by 16 lanes
// (one DPP row; four rows per wave), lane t holding columns 8t .. 8t+7 of
// the batch.  At step i the owner's current value of column i is broadcast
// to the row's 16 lanes (DPP row broadcast, a VALU modifier, so the serial
// chain from one column's error to the next column's value has no LDS
// round trip), which all quantize it identically; the owner keeps code and
// error, and every lane updates its own columns with fma(-err, U[i][col], w)
// (U is zero below the diagonal, so finished columns are left as they are).
// At the start of each group (NVFP4: 16 columns, E4M3 patterns; MXFP4: 32
// columns, E8M0 exponents, no global scale) lane t evaluates the window
// candidate at offset lo + t on the group's current values (the sweep's
// loss), and a (loss, candidate) minimum over the row's lanes picks the
// scale.  The batch's
// scaled errors replace its columns of W for the trailing update.  The
// column loop is unrolled at compile time because the broadcast's source
// lane is an immediate.
constexpr int kGptqBatchThreads = 256;
constexpr int kGptqRowsPerWg = kGptqBatchThreads / 16;

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F &&f) {
  (f(std::integral_constant<int, I>{}), ...);
}

template <bool WMSE, int FMT>
__global__ __launch_bounds__(kGptqBatchThreads) void gptq_batch_kernel(
    float *__restrict__ W, int64_t ld, int rows, int cols, int i1, const float *__restrict__ U,
    const float *__restrict__ imp, const float *__restrict__ gscale, int lo, int hi, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales, uint32_t *__restrict__ status) {
  __shared__ __attribute__((aligned(1024))) float Ub[kGptqBatch][kGptqBatch];
  __shared__ float Vtab[128], Rtab[128], rdiag[kGptqBatch], impb[kGptqBatch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = lane & 15;
  const int r = blockIdx.x * kGptqRowsPerWg + (tid >> 4);
  const bool live = r < rows;  // dead rows still take part in the broadcasts
  constexpr bool MX = FMT == FP4Q_MXFP4;
  const float S = MX ? 1.0f : *gscale;
  const float S_inv = (S == 0.0f) ? 0.0f : 1.0f / S;
  // Every global load is issued before any of them is waited for: the tables, the diagonal and the
  // importance (threads < 128), the row's weights (dead rows read row 0), and the U block into
  // registers, part j holding rows 8j .. 8j+7.  Part j is stored to LDS only when the columns reach
  // row 8j, so the block arrives while the first columns are quantized (the compiler waits for
  // each register's load precisely).
  float tv = 0.0f, trc = 0.0f, dg = 1.0f, im = 1.0f;
  if (tid < 128) {
    tv = kE4M3.v[tid];
    trc = kE4M3.r[tid];
    dg = U[(int64_t)(i1 + tid) * cols + i1 + tid];
    if (WMSE) im = imp[i1 + tid];
  }
  float *wr = W + (int64_t)(live ? r : 0) * ld + i1 + 8 * t;
  const f32x4 wa = *reinterpret_cast<const f32x4 *>(wr);
  const f32x4 wb = *reinterpret_cast<const f32x4 *>(wr + 4);
  f32x4 up[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = tid + kGptqBatchThreads * j;
    up[j] = *reinterpret_cast<const f32x4 *>(U + (int64_t)(i1 + (e >> 5)) * cols + i1 + (e & 31) * 4);
  }
  // part j of the U block to LDS (rows 8j .. 8j+7; element e = tid + 256 j is Ub[e / 32][4 (e % 32)])
  auto stash_u = [&](auto j_c) {
    constexpr int j = decltype(j_c)::value;
    const int e = tid + kGptqBatchThreads * j;
    *reinterpret_cast<f32x4 *>(&Ub[e >> 5][(e & 31) * 4]) = up[j];
  };
  if (tid < 128) {
    Vtab[tid] = tv;
    Rtab[tid] = trc;
    if (!((dg > 0.0f) & (dg <= 3.402823466e38f))) atomicOr(status, FP4Q_DATA_BAD_HESSIAN);
    rdiag[tid] = 1.0f / dg;  // correctly rounded
    impb[tid] = im;
    if (WMSE && !((im >= 0.0f) & (im <= 3.402823466e38f))) atomicOr(status, FP4Q_DATA_BAD_IMPORTANCE);
  }
  stash_u(std::integral_constant<int, 0>{});
  float w[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[k] = live ? wa[k] : 0.0f;
    w[4 + k] = live ? wb[k] : 0.0f;
  }
  if constexpr (MX) {  // no global-max pass checked the weights
    bool finite = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) finite &= fabsf(w[k]) <= 3.402823466e38f;
    if (!finite) atomicOr(status, FP4Q_DATA_NONFINITE_INPUT);
  }
  __syncthreads();  // the tables and rows 0 .. 7 of the U block
  uint32_t code8 = 0;
  float err8[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) err8[k] = 0.0f;
  float V = 1.0f, R = 1.0f;
  f32x4 un0 = *reinterpret_cast<const f32x4 *>(&Ub[0][8 * t]);
  f32x4 un1 = *reinterpret_cast<const f32x4 *>(&Ub[0][8 * t + 4]);
  float rdn = rdiag[0];
  static_for(std::make_integer_sequence<int, 16>{}, [&](auto tt_c) {
    constexpr int tt = decltype(tt_c)::value;
    if constexpr (MX && (tt & 3) == 0) {
      // group [8 tt, 8 tt + 32): its values sit in lanes tt .. tt + 3 of the row
      float z[32], wg[32];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        z[e] = row_bcast<tt>(w[e]);
        z[8 + e] = row_bcast<tt + 1>(w[e]);
        z[16 + e] = row_bcast<tt + 2>(w[e]);
        z[24 + e] = row_bcast<tt + 3>(w[e]);
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) wg[e] = impb[8 * tt + e];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(z[e]));
      const int eb = mx_base_exponent(a);
      const int E = eb + lo + t;
      const bool ok = (t <= hi - lo) & (E >= -127) & (E <= 127);
      const int Ec = min(max(E, -127), 127);
      const float down = pow2f(-Ec), up = pow2f(Ec);
      float y[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) y[e] = z[e] * down;
      // the block's loss: its two 16-element halves, each summed in order, then added
      const float L0 = loss_of_codes<WMSE>(z, wg, cvt8<false>(y, 0u), cvt8<false>(y + 8, 0u), up);
      const float L1 = loss_of_codes<WMSE>(z + 16, wg + 16, cvt8<false>(y + 16, 0u), cvt8<false>(y + 24, 0u), up);
      float Lm = ok ? L0 + L1 : __builtin_inff();
      int em = ok ? E : 0x7FFFFFFF;
      row_argmin16(Lm, em);
      const int es = em == 0x7FFFFFFF ? max(-127, eb + lo) : em;
      V = pow2f(es);
      R = pow2f(-es);
      if (live && t == 0) scales[(int64_t)r * (cols / 32) + ((i1 + 8 * tt) >> 5)] = (uint8_t)(es + 127);
    }
    if constexpr (!MX && (tt & 1) == 0) {
      // group [8 tt, 8 tt + 16): its values sit in lanes tt and tt + 1 of the row
      float us[16], wg[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        us[e] = row_bcast<tt>(w[e]) * S_inv;
        us[8 + e] = row_bcast<tt + 1>(w[e]) * S_inv;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) wg[e] = impb[8 * tt + e];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(us[e]));
      const int base = max(e4m3_rne_sat(a / 6.0f), 1);
      const int p = base + lo + t;
      const bool ok = (t <= hi - lo) & (p >= 1) & (p <= 126);
      const int pc = min(max(p, 1), 126);
      const float Rk = Rtab[pc];
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = us[e] * Rk;
      const float L = loss_of_codes<WMSE>(us, wg, cvt8<false>(y, 0u), cvt8<false>(y + 8, 0u), Vtab[pc]);
      float Lm = ok ? L : __builtin_inff();
      int pm = ok ? p : 0x7FFFFFFF;
      row_argmin16(Lm, pm);
      const int ps = pm == 0x7FFFFFFF ? max(1, base + lo) : pm;
      V = Vtab[ps];
      R = Rtab[ps];
      if (live && t == 0) scales[(int64_t)r * (cols / 16) + ((i1 + 8 * tt) >> 4)] = (uint8_t)ps;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * tt + k;
      // this column's U row was read one column ahead; read the next one now, and keep the reads
      // here (the scheduler would sink them to their use), so their LDS latency stays off the
      // column-to-column chain
      const f32x4 u0 = un0, u1 = un1;
      const float rd = rdn;
      if (i + 1 < kGptqBatch) {
        if (k == 7) {  // the next column opens rows 8 (tt + 1) ..: store them, for every thread
          stash_u(std::integral_constant<int, (tt < 15 ? tt + 1 : 15)>{});
          __syncthreads();
        }
        un0 = *reinterpret_cast<const f32x4 *>(&Ub[i + 1][8 * t]);
        un1 = *reinterpret_cast<const f32x4 *>(&Ub[i + 1][8 * t + 4]);
        rdn = rdiag[i + 1];
      }
      __builtin_amdgcn_sched_barrier(0);
      const float wi = row_bcast<tt>(w[k]);
      const float us_i = wi * S_inv;
      const float y_i = us_i * R;
      // byte 0 holds y_i's code and that of +0 (nibble 0); the other bytes keep the 0 passed in
      const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y_i, 0.0f, 1.0f, 0);
      const float q = fp4x2_to_f32<0>(code).x;  // signed E2M1 value
      const float what = MX ? q * V : (q * V) * S;  // q * V exact; NVFP4: one rounding by S
      const float err = (wi - what) * rd;
      if (t == tt) {
        code8 |= code << (4 * k);
        err8[k] = err;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        w[kk] = fmaf(-err, u0[kk], w[kk]);
        w[4 + kk] = fmaf(-err, u1[kk], w[4 + kk]);
      }
    }
  });
  if (live) {
    *reinterpret_cast<f32x4 *>(wr) = f32x4{err8[0], err8[1], err8[2], err8[3]};
    *reinterpret_cast<f32x4 *>(wr + 4) = f32x4{err8[4], err8[5], err8[6], err8[7]};
    *reinterpret_cast<uint32_t *>(codes + (int64_t)r * (cols / 2) + (i1 + 8 * t) / 2) = code8;
  }
}

// Trailing update W[:, c] -= E * U[i1:i1+kn, c] for the columns c from cbeg
// on (blockIdx.y selects 64 of them), with E = W[:, i1:i1+kn] the scaled
// errors of kn already quantized columns (one batch of 128, or a block of
// 1024): a dense contraction on fp32 MFMA (32x32x2).  A workgroup computes a 64 x 64 tile, each wave a
// 32 x 32 sub-tile whose 16 accumulator rows per lane are read from W at the
// start (their HBM latency then hides behind the contraction instead of
// stalling the epilogue).  E and U are staged through LDS in K chunks of 32:
// E row-major with a padded stride of 33 floats, U k-major, so the stores and
// the operand reads of each k step hit distinct banks.  The k steps run in
// ascending order, so every output element accumulates in the same order.
constexpr int kUpdKc = 32;

__global__ __launch_bounds__(kThreads) void gptq_update_kernel(float *__restrict__ W, int64_t ld, int rows,
                                                               int cols, int i1, int kn, int cbeg,
                                                               const float *__restrict__ U) {
  __shared__ float As[2][64][kUpdKc + 1];
  __shared__ float Bs[2][kUpdKc][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * 64, c0 = cbeg + blockIdx.y * 64;
  const int wr = wave & 1, wc = wave >> 1;
  const int lr = lane & 31, lk = lane >> 5;
  // accumulator v of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l%32
  float cur[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = r0 + wr * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
    cur[v] = row < rows ? W[(int64_t)row * ld + c0 + wc * 32 + lr] : 0.0f;
  }
  // chunk kc of the operands: E rows r0.. (64 x 32, 8 float4 per row), U rows i1 + kc.. (32 x 64)
  f32x4 a[2], b[2];
  auto fetch = [&](int kc) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + kThreads * j;
      const int rr = e >> 3, k4 = e & 7;
      a[j] = (r0 + rr < rows) ? *reinterpret_cast<const f32x4 *>(W + (int64_t)(r0 + rr) * ld + i1 + kc + k4 * 4)
                              : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int kk = e >> 4, j4 = e & 15;
      b[j] = *reinterpret_cast<const f32x4 *>(U + (int64_t)(i1 + kc + kk) * cols + c0 + j4 * 4);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + kThreads * j;
      const int rr = e >> 3, k4 = e & 7;
#pragma unroll
      for (int k = 0; k < 4; ++k) As[buf][rr][k4 * 4 + k] = a[j][k];
      const int kk = e >> 4, j4 = e & 15;
      *reinterpret_cast<f32x4 *>(&Bs[buf][kk][j4 * 4]) = b[j];
    }
  };
  // double-buffered: chunk kc + 1's global loads are in flight while chunk kc's MFMAs run, and one
  // barrier per chunk separates filling one LDS buffer from reading the other
  f32x16 acc = {0};
  fetch(0);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int kc = 0; kc < kn; kc += kUpdKc) {
    const bool more = kc + kUpdKc < kn;
    if (more) fetch(kc + kUpdKc);
#pragma unroll
    for (int k = 0; k < kUpdKc; k += 2) {
      const float av = As[buf][wr * 32 + lr][k + lk];
      const float bv = Bs[buf][k + lk][wc * 32 + lr];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = r0 + wr * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
    if (row < rows) W[(int64_t)row * ld + c0 + wc * 32 + lr] = cur[v] - acc[v];
  }
}

// Decode of an arbitrary E4M3 byte (sign, 0x7F / 0xFF = NaN).
__device__ __forceinline__ float e4m3_decode_any(uint32_t b) {
  const uint32_t m = b & 0x7Fu;
  float v = (m == 0x7Fu) ? __builtin_nanf("") : (m == 0 ? 0.0f : e4m3_value((int)m));
  return (b & 0x80u) ? -v : v;
}

// Magnitude of an E2M1 code index 0..7.
__device__ __forceinline__ float e2m1_magnitude(uint32_t idx) {
  return idx < 2 ? 0.5f * (float)idx : as_f((((idx >> 1) + 126u) << 23) | ((idx & 1u) << 22));
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            const float *__restrict__ gscale, int cpr,
                                                            int cols, int total, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t g0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kThreads + (threadIdx.x & ~63u)));
  int r, c;
  if (!lane_chunk(g0, lane, cpr, total, r, c)) return;
  const uint2 pk = *reinterpret_cast<const uint2 *>(codes + (int64_t)r * (cols / 2) + (int64_t)c * 8);
  float scale, S = 1.0f;
  if constexpr (FMT == FP4Q_NVFP4) {
    scale = e4m3_decode_any(scales[(int64_t)r * cpr + c]);
    S = *gscale;
  } else {
    const uint32_t b = scales[(int64_t)r * (cpr / 2) + (c >> 1)];
    scale = (b == 255u) ? __builtin_nanf("") : pow2f((int)b - 127);
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t code = ((i < 8 ? pk.x : pk.y) >> (4 * (i & 7))) & 0xFu;
    float mag = e2m1_magnitude(code & 7u) * scale;  // exact
    if constexpr (FMT == FP4Q_NVFP4) mag = mag * S;
    v[i] = (code & 8u) ? -mag : mag;
  }
  store_chunk_f32(out + (int64_t)r * cols, c, cpr, lane, v);
}

template <typename T, int HAD>
__global__ __launch_bounds__(kThreads) void hadamard_kernel(const T *__restrict__ x, int64_t ld, int cpr,
                                                             int cols, int total, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t g0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kThreads + (threadIdx.x & ~63u)));
  int r, c;
  // whole groups end together: total is a multiple of HAD/16
  if (!lane_chunk(g0, lane, cpr, total, r, c)) return;
  float z[16];
  load16(x + (int64_t)r * ld + (int64_t)c * 16, z);
  fwht<HAD>(z, lane);
  store_chunk_f32(out + (int64_t)r * cols, c, cpr, lane, z);
}

// ============================================================ dispatch ===

template <typename F>
static void with_had(int n, F &&f) {
  switch (n) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 16: f(std::integral_constant<int, 16>{}); break;
    case 32: f(std::integral_constant<int, 32>{}); break;
    case 64: f(std::integral_constant<int, 64>{}); break;
    default: f(std::integral_constant<int, 128>{}); break;
  }
}

template <typename F>
static void with_dtype(fp4q_dtype_t dt, F &&f) {
  if (dt == FP4Q_BF16) f((const uint16_t *)nullptr);
  else f((const float *)nullptr);
}

static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Rows per wave tile: enough tiles to give every SIMD several waves.  The
// VALU-bound NVFP4 sweep is best near 16 waves of one row per SIMD, the
// memory-bound MXFP4 sweep with as many one-row waves as there are rows.
// The target tile count can be overridden with FP4Q_TILE_TARGET (tuning).
constexpr int64_t kNvTileTarget = 16384;
constexpr int64_t kMxTileTarget = 65536;
static int pick_rows_per_tile(int rows, int nbands, int64_t default_target) {
  const char *now = getenv("FP4Q_TILE_TARGET");
  const int64_t target_tiles = (now && atoi(now) > 0) ? atoi(now) : default_target;
  const int64_t units = (int64_t)rows * nbands;
  int rpt = (int)((units + target_tiles - 1) / target_tiles);
  return rpt < 1 ? 1 : (rpt > 64 ? 64 : rpt);
}

// The GPTQ batches of either format: per 128-column batch the batch kernel,
// then the two-level lazy update (the rest of this block of kGptqBlock
// columns with the batch's 128 error columns; after the block's last batch,
// all later columns with the block's error columns as one contraction).
template <int FMT>
static void gptq_batches(float *w, int64_t rows, int64_t cols, int64_t ld, const float *hinv_chol,
                         const float *importance, const float *global_scale, int off_lo, int off_hi, uint8_t *codes,
                         uint8_t *scales, uint32_t *status, hipStream_t s) {
  const int gb = ceil_div(rows, kGptqRowsPerWg);
  for (int i1 = 0; i1 < cols; i1 += kGptqBatch) {
    if (importance)
      hipLaunchKernelGGL((gptq_batch_kernel<true, FMT>), dim3(gb), dim3(kGptqBatchThreads), 0, s, w, ld, (int)rows,
                         (int)cols, i1, hinv_chol, importance, global_scale, off_lo, off_hi, codes, scales, status);
    else
      hipLaunchKernelGGL((gptq_batch_kernel<false, FMT>), dim3(gb), dim3(kGptqBatchThreads), 0, s, w, ld,
                         (int)rows, (int)cols, i1, hinv_chol, importance, global_scale, off_lo, off_hi, codes, scales,
                         status);
    const int i2 = i1 + kGptqBatch;
    const int b0 = i1 / kGptqBlock * kGptqBlock, b1 = std::min((int)cols, b0 + kGptqBlock);
    if (i2 < b1)
      hipLaunchKernelGGL(gptq_update_kernel, dim3(ceil_div(rows, 64), (b1 - i2) / 64), dim3(kThreads), 0, s, w, ld,
                         (int)rows, (int)cols, i1, kGptqBatch, i2, hinv_chol);
    else if (b1 < cols)
      hipLaunchKernelGGL(gptq_update_kernel, dim3(ceil_div(rows, 64), ((int)cols - b1) / 64), dim3(kThreads), 0, s,
                         w, ld, (int)rows, (int)cols, b0, b1 - b0, b1, hinv_chol);
  }
}

static AmaxOut amax_out(void *workspace, const float *imp, int imp_n) {
  char *b = (char *)workspace;
  return AmaxOut{(uint32_t *)(b + kWsPartials), (uint32_t *)(b + kWsStatus), imp, imp_n};
}

// Global-max pass over x (after the optional rotation): per-workgroup
// maxima into the workspace.  Returns their number.
static int launch_amax(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols, int64_t ld, int hadamard_n,
                       const AmaxOut &ao, hipStream_t s) {
  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  if (hadamard_n == 0 && ld == cols) {
    const int64_t n_vec = rows * cols * (dtype == FP4Q_BF16 ? 2 : 4) / 16;
    const int n = (int)std::min<int64_t>(kAmaxGroups, (n_vec + kThreads * 8 - 1) / (kThreads * 8));
    if (dtype == FP4Q_BF16)
      hipLaunchKernelGGL((amax_flat_kernel<uint16_t>), dim3(n), dim3(kThreads), 0, s, (const u32x4 *)x, n_vec, ao);
    else
      hipLaunchKernelGGL((amax_flat_kernel<float>), dim3(n), dim3(kThreads), 0, s, (const u32x4 *)x, n_vec, ao);
    return n;
  }
  const int n = std::min(kAmaxGroups, ceil_div(total, kThreads * 4));
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    with_had(hadamard_n, [&](auto hc) {
      constexpr int H = decltype(hc)::value;
      if (ld == cols) {
        if constexpr (H != 0)
          hipLaunchKernelGGL((amax_chunks_kernel<T, H>), dim3(n), dim3(kThreads), 0, s, (const T *)x, (int64_t)total,
                             ao);
      } else {
        hipLaunchKernelGGL((amax_kernel<T, H>), dim3(n), dim3(kThreads), 0, s, (const T *)x, ld, cpr, total, ao);
      }
    });
  });
  return n;
}

}  // namespace fp4q

// ============================================================ C ABI ======
using namespace fp4q;

extern "C" {

int fp4q_version(void) { return 100; }

const char *fp4q_status_string(fp4q_status_t s) {
  switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_ERR_NULL: return "a required pointer is NULL";
    case FP4Q_ERR_SHAPE: return "inconsistent shape (rows, cols, ld, block or Hadamard size)";
    case FP4Q_ERR_ARG: return "invalid argument (dtype, loss, window, Hadamard size or flags)";
    case FP4Q_ERR_ALIGN: return "misaligned pointer or row stride (16 bytes required)";
    case FP4Q_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4Q_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

size_t fp4q_workspace_bytes(void) { return kWorkspaceBytes; }

}  // extern "C"

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static fp4q_status_t check_matrix(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                  int block, int hadamard_n) {
  if (dtype != FP4Q_F32 && dtype != FP4Q_BF16) return FP4Q_ERR_ARG;
  if (hadamard_n != 0 && hadamard_n != 16 && hadamard_n != 32 && hadamard_n != 64 && hadamard_n != 128)
    return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols) return FP4Q_ERR_SHAPE;
  if (cols % block) return FP4Q_ERR_SHAPE;
  if (hadamard_n && cols % hadamard_n) return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  const size_t esz = dtype == FP4Q_BF16 ? 2 : 4;
  if (rows > 0 && cols > 0 && (!aligned(x, 16) || (ld * (int64_t)esz) % 16)) return FP4Q_ERR_ALIGN;
  return FP4Q_OK;
}

static fp4q_status_t last_hip_status() {
  return hipGetLastError() == hipSuccess ? FP4Q_OK : FP4Q_ERR_HIP;
}

extern "C" fp4q_status_t fp4q_quantize_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                             int64_t ld, const float *importance, int block,
                                             fp4q_loss_t loss, int off_lo, int off_hi, int hadamard_n,
                                             uint32_t flags, uint8_t *codes, uint8_t *scales,
                                             float *global_scale, float *block_loss, int8_t *offsets,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && (!x || !codes || !scales))) return FP4Q_ERR_NULL;
  if (loss != FP4Q_MSE && loss != FP4Q_WMSE) return FP4Q_ERR_ARG;
  if (loss == FP4Q_WMSE && !importance && !empty) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  if (block != 16) return FP4Q_ERR_SHAPE;
  if (off_lo > 0 || off_hi < 0 || off_lo < -126 || off_hi > 126) return FP4Q_ERR_ARG;
  if (flags & ~FP4Q_GIVEN_SCALE) return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, hadamard_n);
  if (st != FP4Q_OK) return st;
  const bool wmse = loss == FP4Q_WMSE;
  if (!empty && wmse && !aligned(importance, 16)) return FP4Q_ERR_ALIGN;
  if (!empty && (!aligned(codes, 8) || (block_loss && !aligned(block_loss, 4)))) return FP4Q_ERR_ALIGN;

  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  const bool given = flags & FP4Q_GIVEN_SCALE;

  if (rows == 0 || cols == 0) {
    if (!given) hipLaunchKernelGGL(zero_scale_kernel, dim3(1), dim3(1), 0, s, global_scale);
    return last_hip_status();
  }

  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  const int n_partials =
      given ? 0 : launch_amax(x, dtype, rows, cols, ld, hadamard_n, amax_out(workspace, wmse ? importance : nullptr,
                                                                                      (int)cols), s);

  SweepArgs a;
  a.x = x;
  a.ld = ld;
  a.rows = (int)rows;
  a.cols = (int)cols;
  a.cpr = cpr;
  a.imp = wmse ? importance : nullptr;
  a.off_lo = off_lo;
  a.off_hi = off_hi;
  a.nbands = ceil_div(cpr, 64);
  a.rows_per_tile = pick_rows_per_tile((int)rows, a.nbands, kNvTileTarget);
  a.ntiles = a.nbands * ceil_div(rows, a.rows_per_tile);
  a.partials = (const uint32_t *)((const char *)workspace + kWsPartials);
  a.n_partials = n_partials;
  a.check_imp = given;  // else the global-max pass validates the importance
  a.given_scale = given ? global_scale : nullptr;
  a.codes = codes;
  a.scales = scales;
  a.gscale_out = global_scale;
  a.loss = block_loss;
  a.offs = offsets;
  a.status = status;
  const int grid = ceil_div(a.ntiles, kWaves);
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    with_had(hadamard_n, [&](auto hc) {
      constexpr int H = decltype(hc)::value;
      if (wmse)
        hipLaunchKernelGGL((nvfp4_sweep_kernel<T, true, H>), dim3(grid), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((nvfp4_sweep_kernel<T, false, H>), dim3(grid), dim3(kThreads), 0, s, a);
    });
  });
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_global_scale_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                                 int64_t ld, int hadamard_n, float *global_scale, void *workspace,
                                                 size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && !x)) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, 16, hadamard_n);
  if (st != FP4Q_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (empty) {
    hipLaunchKernelGGL(zero_scale_kernel, dim3(1), dim3(1), 0, s, global_scale);
    return last_hip_status();
  }
  // the max pass and the reduction of its partials, as at the start of fp4q_quantize_nvfp4
  const int n_partials = launch_amax(x, dtype, rows, cols, ld, hadamard_n, amax_out(workspace, nullptr, 0), s);
  hipLaunchKernelGGL(scale_from_partials_kernel, dim3(1), dim3(kThreads), 0, s,
                     (const uint32_t *)((const char *)workspace + kWsPartials), n_partials, global_scale,
                     (uint32_t *)((char *)workspace + kWsStatus));
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_quantize_mxfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                             int64_t ld, const float *importance, int block,
                                             fp4q_loss_t loss, int off_lo, int off_hi, int hadamard_n,
                                             uint8_t *codes, uint8_t *scales, float *block_loss,
                                             int8_t *offsets, void *workspace, size_t workspace_bytes,
                                             void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!x || !codes || !scales)) return FP4Q_ERR_NULL;
  if (loss != FP4Q_MSE && loss != FP4Q_WMSE) return FP4Q_ERR_ARG;
  if (loss == FP4Q_WMSE && !importance && !empty) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  if (block != 32) return FP4Q_ERR_SHAPE;
  if (off_lo > 0 || off_hi < 0 || off_lo < -16 || off_hi > 16) return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, hadamard_n);
  if (st != FP4Q_OK) return st;
  const bool wmse = loss == FP4Q_WMSE;
  if (!empty && wmse && !aligned(importance, 16)) return FP4Q_ERR_ALIGN;
  if (!empty && (!aligned(codes, 8) || (block_loss && !aligned(block_loss, 4)))) return FP4Q_ERR_ALIGN;

  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  if (rows == 0 || cols == 0) return FP4Q_OK;

  const int cpr = (int)(cols / 16);
  SweepArgs a;
  a.x = x;
  a.ld = ld;
  a.rows = (int)rows;
  a.cols = (int)cols;
  a.cpr = cpr;
  a.imp = wmse ? importance : nullptr;
  a.off_lo = off_lo;
  a.off_hi = off_hi;
  a.nbands = ceil_div(cpr, 64);
  a.rows_per_tile = pick_rows_per_tile((int)rows, a.nbands, kMxTileTarget);
  a.ntiles = a.nbands * ceil_div(rows, a.rows_per_tile);
  a.partials = nullptr;
  a.n_partials = 0;
  a.check_imp = true;
  a.given_scale = nullptr;
  a.codes = codes;
  a.scales = scales;
  a.gscale_out = nullptr;
  a.loss = block_loss;
  a.offs = offsets;
  a.status = status;
  const int grid = ceil_div(a.ntiles, kWaves);
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    with_had(hadamard_n, [&](auto hc) {
      constexpr int H = decltype(hc)::value;
      if (wmse)
        hipLaunchKernelGGL((mxfp4_sweep_kernel<T, true, H>), dim3(grid), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((mxfp4_sweep_kernel<T, false, H>), dim3(grid), dim3(kThreads), 0, s, a);
    });
  });
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_quantize_relaxed(fp4q_format_t format, const void *x, fp4q_dtype_t dtype,
                                               int64_t rows, int64_t cols, int64_t ld, const uint8_t *scales,
                                               const float *global_scale, const uint16_t *coeffs,
                                               int sub_block, uint8_t *codes, float *dequant_out,
                                               void *workspace, size_t workspace_bytes, void *stream) {
  if (format != FP4Q_NVFP4 && format != FP4Q_MXFP4) return FP4Q_ERR_ARG;
  const int block = format == FP4Q_NVFP4 ? 16 : 32;
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!x || !scales || !codes)) return FP4Q_ERR_NULL;
  if (!empty && format == FP4Q_NVFP4 && !global_scale) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  if (sub_block != 4 && sub_block != 8 && sub_block != 16 && !(sub_block == 32 && block == 32))
    return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, 0);
  if (st != FP4Q_OK) return st;
  if (empty) return FP4Q_OK;
  if (!aligned(codes, 8) || (dequant_out && !aligned(dequant_out, 16)) || (coeffs && !aligned(coeffs, 2)))
    return FP4Q_ERR_ALIGN;
  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  const int grid = ceil_div(total, kThreads);
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    auto go = [&](auto fmt_c, auto sub_c) {
      constexpr int FM = decltype(fmt_c)::value, SB = decltype(sub_c)::value;
      hipLaunchKernelGGL((relaxed_quant_kernel<T, FM, SB>), dim3(grid), dim3(kThreads), 0, s, (const T *)x, ld,
                         cpr, (int)cols, total, scales, global_scale, coeffs, codes, dequant_out, status);
    };
    auto with_sub = [&](auto fmt_c) {
      switch (sub_block) {
        case 4: go(fmt_c, std::integral_constant<int, 4>{}); break;
        case 8: go(fmt_c, std::integral_constant<int, 8>{}); break;
        case 16: go(fmt_c, std::integral_constant<int, 16>{}); break;
        default:
          if constexpr (decltype(fmt_c)::value == FP4Q_MXFP4) go(fmt_c, std::integral_constant<int, 32>{});
          break;
      }
    };
    if (format == FP4Q_NVFP4)
      with_sub(std::integral_constant<int, FP4Q_NVFP4>{});
    else
      with_sub(std::integral_constant<int, FP4Q_MXFP4>{});
  });
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_gptq_nvfp4(float *w, int64_t rows, int64_t cols, int64_t ld,
                                         const float *hinv_chol, const float *importance, int off_lo,
                                         int off_hi, uint32_t flags, uint8_t *codes, uint8_t *scales,
                                         float *global_scale, void *workspace, size_t workspace_bytes,
                                         void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && (!w || !hinv_chol || !codes || !scales))) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  if (off_lo > 0 || off_hi < 0 || off_hi - off_lo > 15) return FP4Q_ERR_ARG;
  if (flags & ~FP4Q_GIVEN_SCALE) return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols || cols % kGptqBatch) return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (empty) return FP4Q_OK;
  if (!aligned(w, 16) || ld % 4 || !aligned(hinv_chol, 16) || !aligned(codes, 4) ||
      (importance && !aligned(importance, 4)))
    return FP4Q_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  const bool given = flags & FP4Q_GIVEN_SCALE;
  if (!given) {
    uint32_t *partials = (uint32_t *)((char *)workspace + kWsPartials);
    const int n_partials = launch_amax(w, FP4Q_F32, rows, cols, ld, 0, amax_out(workspace, nullptr, 0), s);
    hipLaunchKernelGGL(scale_from_partials_kernel, dim3(1), dim3(kThreads), 0, s, partials, n_partials,
                       global_scale, status);
  }
  gptq_batches<FP4Q_NVFP4>(w, rows, cols, ld, hinv_chol, importance, global_scale, off_lo, off_hi, codes, scales,
                           status, s);
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_gptq_mxfp4(float *w, int64_t rows, int64_t cols, int64_t ld,
                                         const float *hinv_chol, const float *importance, int off_lo,
                                         int off_hi, uint8_t *codes, uint8_t *scales, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!w || !hinv_chol || !codes || !scales)) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes) return FP4Q_ERR_WORKSPACE;
  if (off_lo > 0 || off_hi < 0 || off_hi - off_lo > 15) return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols || cols % kGptqBatch) return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (empty) return FP4Q_OK;
  if (!aligned(w, 16) || ld % 4 || !aligned(hinv_chol, 16) || !aligned(codes, 4) ||
      (importance && !aligned(importance, 4)))
    return FP4Q_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  gptq_batches<FP4Q_MXFP4>(w, rows, cols, ld, hinv_chol, importance, nullptr, off_lo, off_hi, codes, scales,
                           status, s);
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_dequantize(fp4q_format_t format, const uint8_t *codes, const uint8_t *scales,
                                         const float *global_scale, int64_t rows, int64_t cols, int block,
                                         float *out, void *stream) {
  if (format != FP4Q_NVFP4 && format != FP4Q_MXFP4) return FP4Q_ERR_ARG;
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!codes || !scales || !out)) return FP4Q_ERR_NULL;
  if (!empty && format == FP4Q_NVFP4 && !global_scale) return FP4Q_ERR_NULL;
  if (block != (format == FP4Q_NVFP4 ? 16 : 32)) return FP4Q_ERR_SHAPE;
  if (rows < 0 || cols < 0 || cols % block) return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (empty) return FP4Q_OK;
  if (!aligned(codes, 8) || !aligned(out, 16)) return FP4Q_ERR_ALIGN;
  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  hipStream_t s = (hipStream_t)stream;
  const int grid = ceil_div(total, kThreads);
  if (format == FP4Q_NVFP4)
    hipLaunchKernelGGL((dequant_kernel<FP4Q_NVFP4>), dim3(grid), dim3(kThreads), 0, s, codes, scales,
                       global_scale, cpr, (int)cols, total, out);
  else
    hipLaunchKernelGGL((dequant_kernel<FP4Q_MXFP4>), dim3(grid), dim3(kThreads), 0, s, codes, scales,
                       global_scale, cpr, (int)cols, total, out);
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_block_hadamard(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                             int64_t ld, int n, float *out, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!x || !out)) return FP4Q_ERR_NULL;
  if (n == 0) return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, 16, n);
  if (st != FP4Q_OK) return st;
  if (empty) return FP4Q_OK;
  if (!aligned(out, 16)) return FP4Q_ERR_ALIGN;
  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  hipStream_t s = (hipStream_t)stream;
  const int grid = ceil_div(total, kThreads);
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    with_had(n, [&](auto hc) {
      constexpr int H = decltype(hc)::value;
      if constexpr (H != 0)
        hipLaunchKernelGGL((hadamard_kernel<T, H>), dim3(grid), dim3(kThreads), 0, s, (const T *)x, ld, cpr,
                           (int)cols, total, out);
    });
  });
  return last_hip_status();
}
