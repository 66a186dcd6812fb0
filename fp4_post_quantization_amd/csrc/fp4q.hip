// fp4q: FP4 microscaling block quantization with block-scale search for
// gfx950 (MI355X).  Kernels and the C ABI declared in include/fp4q.h.
//
// Work decomposition: a lane owns 16 contiguous elements of a row ("chunk"),
// an n-point Hadamard group n/16 adjacent lanes; an NVFP4 block is one lane.
// The MXFP4 sweep gives a lane a whole 32-element block instead.  Block
// losses are accumulated inside the lane, so the candidate sweep needs no
// LDS traffic for data and no barriers.
//
// The quantize kernels map a wave to a tile of 64 consecutive lane units of
// a column band times a few rows; the per-column importance of WMSE is
// loaded into registers once per tile and reused for every row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
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

// The dispatch ID of the running kernel: the index of its packet in the
// hardware queue, the same in every workgroup of a launch and different for
// every launch on the queue.
extern "C" __device__ unsigned long long fp4q_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// The status word of a call is a 64-bit slot at the start of the workspace:
// its low half (byte 0) holds the FP4Q_DATA_* bits, its high half the low
// 32 bits of the dispatch ID of the call's first kernel.  That kernel's
// workgroups merge into the slot by compare-and-swap.  A slot with another
// tag belongs to an earlier call, or is garbage, and is replaced; a slot
// with this call's tag gets the bits ORed in.  So in whichever order the
// workgroups arrive, the slot ends with this call's tag and exactly the
// bits its kernels reported.  Workgroup 0 of the first kernel always merges
// (with no bits if it has none), so a call without errors still replaces
// the slot; nothing waits on anything.  The call's later kernels run after
// the first on the stream and OR their bits into the low half.
struct Status {
  uint32_t *slot;
  bool first;  // this kernel is the call's first: merge under its dispatch tag

  __device__ void merge(uint32_t bits) const {
    unsigned long long *p = reinterpret_cast<unsigned long long *>(slot);
    const unsigned long long tag = (unsigned long long)(uint32_t)fp4q_dispatch_id() << 32;
    unsigned long long old = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
      const unsigned long long keep = (old & 0xFFFFFFFF00000000ull) == tag ? (old & 0xFFFFFFFFull) : 0ull;
      const unsigned long long want = tag | keep | bits;
      if (want == old) return;
      const unsigned long long seen = atomicCAS(p, old, want);
      if (seen == old) return;
      old = seen;
    }
  }
  // an error found by any workgroup
  __device__ void report(uint32_t bits) const {
    if (first) merge(bits);
    else atomicOr(slot, bits);
  }
  // at the start of a kernel: workgroup 0 of the call's first kernel takes the slot
  __device__ void begin() const {
    if (first && blockIdx.x == 0 && threadIdx.x == 0) merge(0u);
  }
  // at the end of a kernel whose lanes gathered their error bits in err: one report site for all
  // of them (thread 0 of workgroup 0 reports even without errors, taking the slot for a first kernel)
  __device__ void finish(uint32_t err) const {
    if (__builtin_expect(err != 0u, 0) || (first && blockIdx.x == 0 && threadIdx.x == 0)) report(err);
  }
};

// The only kernel of an empty call: takes the status slot for the call, or
// adds to it (first = false), with no bits or those of validating a given
// NVFP4 global scale, and optionally writes the global scale of an empty
// NVFP4 tensor (0).
__global__ __launch_bounds__(64) void status_init_kernel(uint32_t *__restrict__ status, bool first,
                                                          const float *__restrict__ given_scale,
                                                          float *__restrict__ zero_scale_out) {
  if (threadIdx.x == 0) {
    uint32_t bits = 0u;
    if (given_scale) {
      const float S = *given_scale;
      if (!(S >= 0.0f) || isinf(S)) bits |= FP4Q_DATA_BAD_GLOBAL_SCALE;
    }
    if (zero_scale_out) *zero_scale_out = 0.0f;
    const Status st{status, first};
    if (first) st.merge(bits);
    else if (bits) st.report(bits);
  }
}

// Where the global-max pass puts its results.
struct AmaxOut {
  uint32_t *partials;  // [gridDim.x] per-workgroup maxima
  uint32_t *status;
  const float *imp;    // importance [imp_n] to validate, or null
  int imp_n;
  bool first;          // the call's first kernel: takes the status slot (else the call adds to it)
};

// Bit 31 of a max-pass partial (the maxima are |x| bit patterns, below
// 2^31): its workgroup found a bad importance entry.
constexpr uint32_t kPartialBadImp = 0x80000000u;

// End of a global-max pass, the first kernel of its call: m is this
// thread's maximum |bits|; the workgroup's maximum goes to
// partials[blockIdx.x].  The workgroups also validate the importance vector
// between them (a strided slice each), so the quantizer that follows need
// not, and report it in bit 31 of their partial.  No workgroup touches the
// status slot except workgroup 0, which takes it for the call (unless the
// call adds to it); the kernel that reduces the partials sets its bits.
__device__ void finish_amax(uint32_t m, const AmaxOut &o) {
  __shared__ uint32_t red[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bool ok = true;
  if (o.imp) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < o.imp_n; i += (int64_t)gridDim.x * kThreads)
      ok &= (o.imp[i] >= 0.0f) & (o.imp[i] <= 3.402823466e38f);
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  const int bad_imp = __syncthreads_or(!ok);
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = red[k] > r ? red[k] : r;
    o.partials[blockIdx.x] = r | (bad_imp ? kPartialBadImp : 0u);
    if (blockIdx.x == 0 && o.first) Status{o.status, true}.merge(0u);
  }
}

// Reduction of the max-pass partials by one wave: the maximum |x| bit
// pattern and the status bits the partials carry.
__device__ __forceinline__ uint32_t reduce_partials(const uint32_t *partials, int n, int lane, uint32_t &bits) {
  uint32_t m = 0, f = 0;
  for (int i = lane; i < n; i += 64) {
    const uint32_t v = partials[i];
    m = max(m, v & ~kPartialBadImp);
    f |= v;
  }
  m = wave_max_u32(m);
  const bool bad_imp = __ballot((f & kPartialBadImp) != 0) != 0;  // one wave-wide test, no shuffles
  bits = (m >= 0x7F800000u ? FP4Q_DATA_NONFINITE_INPUT : 0u) | (bad_imp ? FP4Q_DATA_BAD_IMPORTANCE : 0u);
  return m;
}

// Per-workgroup maximum of |x| (after the optional rotation) as a float32
// bit pattern.  Integer order of |bits| is float order for finite values,
// and any Inf/NaN yields a pattern >= 0x7F800000.
template <typename T, int HAD>
__global__ __launch_bounds__(kThreads) void amax_kernel(const T *__restrict__ x, int64_t ld, int cpr,
                                                         int total, AmaxOut o) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += stride) {
    const int64_t r = g / cpr, c = g - r * cpr;
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
  int rows, cols, cpr;          // cpr = lane units per row: 16-column chunks (NVFP4), 32-column blocks (MXFP4)
  const float *imp;             // [cols] or null
  int off_lo, off_hi;
  int rows_per_tile, nbands, ntiles;
  const uint32_t *partials;     // amax partials (NVFP4, computed scale)
  int n_partials;
  const float *given_scale;     // NVFP4 with FP4Q_GIVEN_SCALE, else null
  bool check_inputs;            // validate the importance and a given scale here (no max pass did)
  bool status_first;            // this sweep is the call's first kernel (takes the status slot)
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

// Loss of one candidate over 16 elements from their codes: e_i =
// fp32(us_i - q_i*V), summed in element order with one rounding per term,
// acc <- fma(t_i, e_i, acc), t_i = e_i (MSE) or fp32(w_i * e_i) (WMSE),
// starting from acc0 (0 for a block's first 16 elements; a 32-element block
// continues its first half's sum).  us and q carry the sign of x (the
// conversions are sign-symmetric), so e_i is the error up to its sign and
// t_i * e_i is unchanged; q*V is exact, so fmaf(-q, V, us) is exactly
// fp32(us - q*V).
template <bool WMSE>
__device__ __forceinline__ float loss_of_codes(const float us[16], const float w[16], uint32_t pk0,
                                               uint32_t pk1, float V, float acc0 = 0.0f) {
  float q[16];
  fp4x8_to_f32(pk0, q);
  fp4x8_to_f32(pk1, q + 8);
  float acc = acc0;
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
  const Status st{a.status, a.status_first};
  uint32_t err = 0u;  // this lane's data errors, reported once at the end
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
      if (a.check_inputs && blockIdx.x == 0 && lane == 0 && (!(S >= 0.0f) || isinf(S)))
        err |= FP4Q_DATA_BAD_GLOBAL_SCALE;
    } else {
      uint32_t bits;
      const uint32_t m = reduce_partials(a.partials, a.n_partials, lane, bits);
      S = as_f(m) / 1536.0f;  // max|x| / (256 * 6), correctly rounded
      if (blockIdx.x == 0 && lane == 0) {
        *a.gscale_out = S;
        err |= bits;
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
  if (!active) return;  // thread 0 of workgroup 0 (tile 0, chunk 0) is always active
  if constexpr (WMSE) {
    if (a.check_inputs && !importance_ok(w)) err |= FP4Q_DATA_BAD_IMPORTANCE;
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
      if (!finite) err |= FP4Q_DATA_NONFINITE_INPUT;
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
  st.finish(err);
}

// Loss of one candidate over a lane's 32-element MXFP4 block from its four
// code words: one in-order chain over all 32 elements.
template <bool WMSE>
__device__ __forceinline__ float loss_of_codes32(const float z[32], const float w[32], const uint32_t k[4], float V) {
  return loss_of_codes<WMSE>(z + 16, w + 16, k[2], k[3], V, loss_of_codes<WMSE>(z, w, k[0], k[1], V));
}

// MXFP4 exponent sweep for one block (this lane's 32 elements): exponents E
// and E + 1 pair up, E + 1 converted from the products of E with the halving
// scale (8 products at a time, each converted for both members).  Returns
// E*; Lbest gets its loss and, KEEP, kb its codes.
template <bool WMSE, bool KEEP>
__device__ __forceinline__ int mx_sweep(const float z[32], const float w[32], int eb, int lo, int hi, float &Lbest,
                                        uint32_t kb[4]) {
  Lbest = __builtin_inff();
  int ebest = max(-127, eb + lo);
  uint32_t k[4] = {0u, 0u, 0u, 0u}, h[4] = {0u, 0u, 0u, 0u};
  for (int o = lo; o <= hi; o += 2) {
    const int E = eb + o;
    const bool ok = (E >= -127) & (E <= 127);
    const int Ec = min(max(E, -127), 127);
    const float down = pow2f(-Ec);
    const bool pair = o + 1 <= hi;
    const bool exact_half = E >= -127;  // else the lower member is clamped: convert E + 1 directly
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = z[8 * j + i] * down;
      k[j] = cvt8<false>(y, k[j]);
      if (pair & exact_half) h[j] = cvt8<true>(y, h[j]);
    }
    if (pair) {
      const int E1 = E + 1;
      const bool ok1 = (E1 >= -127) & (E1 <= 127);
      const int E1c = min(max(E1, -127), 127);
      if (!exact_half) {
        const float d1 = pow2f(-E1c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float y[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = z[8 * j + i] * d1;
          h[j] = cvt8<false>(y, h[j]);
        }
      }
      const bool t1 = consider(loss_of_codes32<WMSE>(z, w, h, pow2f(E1c)), E1, ok1, Lbest, ebest);
      if constexpr (KEEP) {
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[j] = t1 ? h[j] : kb[j];
      }
    }
    const bool t0 = consider(loss_of_codes32<WMSE>(z, w, k, pow2f(Ec)), E, ok, Lbest, ebest);
    if constexpr (KEEP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) kb[j] = t0 ? k[j] : kb[j];
    }
  }
  return ebest;
}

// Sylvester block Hadamard for lanes that own 32 elements: stages h = 1 ..
// min(N, 32)/2 inside the lane (two independent 16-groups when N = 16), then
// h = 32 and 64 with the partner lanes l ^ 1 and l ^ 2 (N = 64, 128), in the
// oracle's stage order, then the scaling by fp32(1/sqrt(N)).
template <int N>
__device__ __forceinline__ void fwht32(float z[32], int lane) {
  constexpr int HM = N < 32 ? N : 32;
#pragma unroll
  for (int h = 1; h < HM; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        float a = z[i], b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
  if constexpr (N >= 64) {
    const bool hi = lane & 1;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float o = xor_lane<1>(z[i]);
      z[i] = hi ? (o - z[i]) : (z[i] + o);
    }
  }
  if constexpr (N >= 128) {
    const bool hi = lane & 2;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float o = xor_lane<2>(z[i]);
      z[i] = hi ? (o - z[i]) : (z[i] + o);
    }
  }
  const float c = hadamard_scale<N>();
#pragma unroll
  for (int i = 0; i < 32; ++i) z[i] = z[i] * c;
}

// A wave's row segment for the MXFP4 sweep (64 blocks of 32 elements, NP
// 16-byte pieces per block) is read with fully coalesced loads (lane l takes
// piece 64k + l in load k), stored in LDS block by block with one piece of
// padding (so both the stores and the lanes' reads of their own blocks
// spread over the banks), and read back as each lane's own block.
template <typename T>
struct MxStage {
  static constexpr int NP = 2 * (int)sizeof(T);  // 4 (bf16) or 8 (float32)
  u32x4 q[64 * (NP + 1)];
};

// The 32 elements of a block from its NP pieces, widened to float32.
__device__ __forceinline__ void widen_block(const u32x4 (&p)[4], float z[32]) {  // bf16
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t w = p[k >> 2][k & 3];
    z[2 * k] = as_f(w << 16);
    z[2 * k + 1] = as_f(w & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen_block(const u32x4 (&p)[8], float z[32]) {  // float32
#pragma unroll
  for (int k = 0; k < 32; ++k) z[k] = as_f(p[k >> 2][k & 3]);
}

// MXFP4 exponent sweep: one lane per 32-element block (a.cpr counts blocks
// here), so a block's loss is one in-lane chain and its maximum needs no
// exchange.  Exponents E and E + 1 form pairs: fp32(x * 2^-(E+1)) =
// fp32(x * 2^-E) / 2.
template <typename T, bool WMSE, int HAD>
__global__ __launch_bounds__(kThreads) void mxfp4_sweep_kernel(SweepArgs a) {
  constexpr int NP = MxStage<T>::NP;
  __shared__ MxStage<T> stage[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int tile = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wave);
  if (tile >= a.ntiles) return;
  const int band = tile % a.nbands, rg = tile / a.nbands;
  const int b = band * 64 + lane;
  // every lane takes part in the loads and the staging; only lanes on a block store results (a
  // Hadamard group's lanes agree, since cols is a multiple of HAD)
  const bool active = b < a.cpr;
  const int npieces = min(64, a.cpr - band * 64) * NP;  // pieces of this band's segment
  const int r0 = rg * a.rows_per_tile;
  const int r1 = min(a.rows, r0 + a.rows_per_tile);
  u32x4 *st = stage[wave].q;
  const Status status{a.status, a.status_first};
  uint32_t err = 0u;  // this lane's data errors, reported once at the end

  float w[32];
  if constexpr (WMSE) {
    if (active) {
      load_importance(a.imp + (int64_t)b * 32, w);
      load_importance(a.imp + (int64_t)b * 32 + 16, w + 16);
      if (a.check_inputs && !(importance_ok(w) & importance_ok(w + 16))) err |= FP4Q_DATA_BAD_IMPORTANCE;
    }
  }

  const char *seg = static_cast<const char *>(a.x) + (int64_t)band * 64 * 32 * (int64_t)sizeof(T);
  const int64_t row_bytes = a.ld * (int64_t)sizeof(T);
  auto load_row = [&](int r, u32x4 (&d)[NP]) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(seg + (int64_t)r * row_bytes);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int g = 64 * k + lane;
      d[k] = g < npieces ? __builtin_nontemporal_load(src + g) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const int lo = a.off_lo, hi = a.off_hi;
  // short windows keep the winner's codes (selects per candidate) instead of converting again
  const bool keep = hi - lo < 8;
  u32x4 cur[NP], nxt[NP];
  load_row(r0, cur);
  for (int r = r0; r < r1; ++r) {
    if (r + 1 < r1) load_row(r + 1, nxt);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int g = 64 * k + lane;
      st[(g / NP) * (NP + 1) + g % NP] = cur[k];
    }
    // lanes read what other lanes of the same wave wrote: LDS operations of a wave complete in order
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    u32x4 mine[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) mine[j] = st[lane * (NP + 1) + j];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float z[32];
    widen_block(mine, z);
    if constexpr (HAD != 0) fwht32<HAD>(z, lane);

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(z[i]));
    const int eb = mx_base_exponent(amax);

    float Lbest;
    uint32_t kb[4] = {0u, 0u, 0u, 0u};  // codes of the best candidate (short windows)
    const int ebest = keep ? mx_sweep<WMSE, true>(z, w, eb, lo, hi, Lbest, kb)
                           : mx_sweep<WMSE, false>(z, w, eb, lo, hi, Lbest, kb);

    // A non-finite element makes its e, and so every candidate's loss, NaN or infinite (the terms
    // t * e are never negative), so a finite best loss proves the block finite; the elementwise
    // test runs only when it is not (an overflowing loss of finite data also lands there).
    const bool lfin = Lbest <= 3.402823466e38f;
    if (!lfin) {
      bool finite = true;
#pragma unroll
      for (int i = 0; i < 32; ++i) finite &= fabsf(z[i]) <= 3.402823466e38f;
      if (!finite && active) err |= FP4Q_DATA_NONFINITE_INPUT;
    }
    if (!(keep & lfin)) {  // else the winner's codes were kept
      const float db = pow2f(-ebest);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = z[8 * j + i] * db;
        kb[j] = cvt8<false>(y, 0u);
      }
    }
    if (active) {
      uint2 *cp = reinterpret_cast<uint2 *>(a.codes + (int64_t)r * (a.cols / 2) + (int64_t)b * 16);
      cp[0] = make_uint2(kb[0], kb[1]);
      cp[1] = make_uint2(kb[2], kb[3]);
      const int64_t bi = (int64_t)r * a.cpr + b;
      a.scales[bi] = (uint8_t)(ebest + 127);
      if (a.loss) a.loss[bi] = Lbest;
      if (a.offs) a.offs[bi] = (int8_t)(ebest - eb);
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) cur[k] = nxt[k];
  }
  status.finish(err);  // thread 0 of workgroup 0 (tile 0) gets here
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
                                                                  float *__restrict__ dq, Status status) {
  const int lane = threadIdx.x & 63;
  uint32_t err = 0u;  // this lane's data errors, reported once at the end
  if constexpr (FMT == FP4Q_NVFP4) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      const float Sg = *gscale;
      if (!(Sg >= 0.0f) || isinf(Sg)) err |= FP4Q_DATA_BAD_GLOBAL_SCALE;
    }
  }
  const int64_t g0 = (int64_t)blockIdx.x * kThreads + 64 * wave_index();
  int r, c;
  if (!lane_chunk(g0, lane, cpr, total, r, c)) return;  // thread 0 of workgroup 0 never returns here
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
  err |= (bad ? FP4Q_DATA_BAD_SCALE : 0u) | (finite ? 0u : FP4Q_DATA_NONFINITE_INPUT);
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
  status.finish(err);
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
  if (threadIdx.x < 64) {
    uint32_t bits;
    const uint32_t m = reduce_partials(partials, n, threadIdx.x, bits);
    if (threadIdx.x == 0) {
      *gscale = as_f(m) / 1536.0f;
      if (bits) atomicOr(status, bits);
    }
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

// partials (NVFP4, the call's first batch when a max pass ran): every workgroup takes S from the max
// pass's per-workgroup maxima itself, and workgroup 0 writes it to gscale for the later batches.
// Win / ldin: where the batch's columns are read (W, or the caller's weight when no update has
// touched them yet); W is where its errors go.  pk >= 0: first apply the errors of the 128 columns
// at pk (the previous batch, in W) to this batch's columns, for the workgroup's own rows: a
// 16 x 128 x 128 contraction on fp32 MFMA (16x16x4) in place of a launch of the near update.
//
// GIVEN (static reordering): the batch's columns are processing slots i1 .. i1 + 127 of the order perm,
// and every group's scale is fixed already: slot j of row r is rounded at the scale byte of its stored
// group, scales[r][perm[j] / block] (row-major, cols / block bytes per row), read here and not
// written.  The sweep at group starts is skipped; codes go to slot j's position in `codes`.
template <bool WMSE, int FMT, bool GIVEN = false>
__global__ __launch_bounds__(kGptqBatchThreads) void gptq_batch_kernel(
    float *W, int64_t ld, const float *Win, int64_t ldin, int pk, int rows, int cols, int i1,
    const float *__restrict__ U,
    const float *__restrict__ imp, float *__restrict__ gscale, const uint32_t *__restrict__ partials,
    int n_partials, int lo, int hi, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, Status status,
    const int32_t *__restrict__ perm = nullptr) {
  __shared__ __attribute__((aligned(1024))) float Ub[kGptqBatch][kGptqBatch];
  __shared__ float Vtab[128], Rtab[128], rdiag[kGptqBatch], impb[kGptqBatch];
  __shared__ float Pe[kGptqRowsPerWg][kGptqBatch + 4];  // pk >= 0: the rows' errors, then the update
  // GIVEN: each row's value and reciprocal of its fixed scale for every column of the batch
  __shared__ float Vg[GIVEN ? kGptqRowsPerWg : 1][GIVEN ? kGptqBatch : 1];
  __shared__ float Rg[GIVEN ? kGptqRowsPerWg : 1][GIVEN ? kGptqBatch : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = lane & 15;
  const int r = blockIdx.x * kGptqRowsPerWg + (tid >> 4);
  const bool live = r < rows;  // dead rows still take part in the broadcasts
  constexpr bool MX = FMT == FP4Q_MXFP4;
  float S = 1.0f;
  if (!MX && partials) {
    uint32_t bits;
    S = as_f(reduce_partials(partials, n_partials, lane, bits)) / 1536.0f;
    if (blockIdx.x == 0 && tid == 0) {
      *gscale = S;
      if (bits) status.report(bits);
    }
  } else if (!MX) {
    S = *gscale;
  }
  const float S_inv = (S == 0.0f) ? 0.0f : 1.0f / S;
  // Every global load is issued before any of them is waited for: the tables, the diagonal and the
  // importance (threads < 128), the row's weights (dead rows read row 0), and the U block into
  // registers, part j holding rows 8j .. 8j+7.  The whole block goes to LDS before the column loop
  // (after the single-panel update, which uses the same LDS): storing part j only when the columns
  // reach row 8j hid some load latency but cost a barrier every 8 columns, measured 4% slower.
  float tv = 0.0f, trc = 0.0f, dg = 1.0f, im = 1.0f;
  if (tid < 128) {
    tv = kE4M3.v[tid];
    trc = kE4M3.r[tid];
    dg = U[(int64_t)(i1 + tid) * cols + i1 + tid];
    if (WMSE) im = imp[i1 + tid];
  }
  status.begin();
  // a given NVFP4 scale is checked once, by the call's first kernel
  if (!MX && status.first && blockIdx.x == 0 && tid == 0 && (!(S >= 0.0f) || isinf(S)))
    status.report(FP4Q_DATA_BAD_GLOBAL_SCALE);
  float *wr = W + (int64_t)(live ? r : 0) * ld + i1 + 8 * t;
  const float *wsrc = Win + (int64_t)(live ? r : 0) * ldin + i1 + 8 * t;
  const f32x4 wa = *reinterpret_cast<const f32x4 *>(wsrc);
  const f32x4 wb = *reinterpret_cast<const f32x4 *>(wsrc + 4);
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
    if (!((dg > 0.0f) & (dg <= 3.402823466e38f))) status.report(FP4Q_DATA_BAD_HESSIAN);
    rdiag[tid] = 1.0f / dg;  // correctly rounded
    impb[tid] = im;
    if (WMSE && !((im >= 0.0f) & (im <= 3.402823466e38f))) status.report(FP4Q_DATA_BAD_IMPORTANCE);
  }
  float w[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[k] = live ? wa[k] : 0.0f;
    w[4 + k] = live ? wb[k] : 0.0f;
  }
  if (pk >= 0) {
    // the rows' errors at pk into Pe, U[pk .. pk + 128][i1 .. i1 + 128] into Ub (free until part 0
    // of this batch's own U block is stored below)
    const float *er = W + (int64_t)(live ? r : 0) * ld + pk + 8 * t;
    *reinterpret_cast<f32x4 *>(&Pe[tid >> 4][8 * t]) = *reinterpret_cast<const f32x4 *>(er);
    *reinterpret_cast<f32x4 *>(&Pe[tid >> 4][8 * t + 4]) = *reinterpret_cast<const f32x4 *>(er + 4);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = tid + kGptqBatchThreads * j;
      *reinterpret_cast<f32x4 *>(&Ub[e >> 5][(e & 31) * 4]) =
          *reinterpret_cast<const f32x4 *>(U + (int64_t)(pk + (e >> 5)) * cols + i1 + (e & 31) * 4);
    }
    __syncthreads();
    // wave v: columns 32 v .. 32 v + 31 as two 16 x 16 blocks; lane l supplies A[l % 16][k = l / 16]
    // and B[k = l / 16][l % 16] of each k step of 4, and holds D[4 (l / 16) + i][l % 16] in register i
    const int wv = tid >> 6, li = lane & 15, lq = lane >> 4;
    f32x4 d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int k = 0; k < kGptqBatch; k += 4) {
      const float a = Pe[li][k + lq];
      d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Ub[k + lq][32 * wv + li], d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Ub[k + lq][32 * wv + 16 + li], d1, 0, 0, 0);
    }
    __syncthreads();  // every wave is done with Pe and Ub
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Pe[4 * lq + i][32 * wv + li] = d0[i];
      Pe[4 * lq + i][32 * wv + 16 + li] = d1[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = w[k] - Pe[tid >> 4][8 * t + k];
  }
  static_for(std::make_integer_sequence<int, 16>{}, [&](auto j_c) { stash_u(j_c); });
  if constexpr (GIVEN) {
    // lane t of a row: the scales of the batch's columns 8t .. 8t+7 (perm entries were range-checked by
    // the call's first kernel; clamped here all the same)
    constexpr int kBlk = FMT == FP4Q_MXFP4 ? 32 : 16;
    const uint8_t *srow = scales + (int64_t)(live ? r : 0) * (cols / kBlk);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = min(max(perm[i1 + 8 * t + k], 0), cols - 1);
      const int b = srow[c / kBlk];
      float v, rc;
      if constexpr (FMT == FP4Q_MXFP4) {
        v = pow2f(b - 127);
        rc = pow2f(127 - b);
      } else {
        const int pc = min(max(b, 1), 126);
        v = kE4M3.v[pc];
        rc = kE4M3.r[pc];
      }
      Vg[tid >> 4][8 * t + k] = v;
      Rg[tid >> 4][8 * t + k] = rc;
    }
  }
  {  // MXFP4 and NVFP4 with a given scale run no global-max pass over the weights
    bool finite = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) finite &= fabsf(w[k]) <= 3.402823466e38f;
    if (!finite) status.report(FP4Q_DATA_NONFINITE_INPUT);
  }
  __syncthreads();  // the tables and the U block
  uint32_t code8 = 0;
  float err8[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) err8[k] = 0.0f;
  float V = 1.0f, R = 1.0f;
  float vgn = GIVEN ? Vg[GIVEN ? tid >> 4 : 0][0] : 1.0f, rgn = GIVEN ? Rg[GIVEN ? tid >> 4 : 0][0] : 1.0f;
  f32x4 un0 = *reinterpret_cast<const f32x4 *>(&Ub[0][8 * t]);
  f32x4 un1 = *reinterpret_cast<const f32x4 *>(&Ub[0][8 * t + 4]);
  float rdn = rdiag[0];
  static_for(std::make_integer_sequence<int, 16>{}, [&](auto tt_c) {
    constexpr int tt = decltype(tt_c)::value;
    if constexpr (!GIVEN && MX && (tt & 3) == 0) {
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
      // the block's loss: one in-order chain over its 32 elements
      const uint32_t kc[4] = {cvt8<false>(y, 0u), cvt8<false>(y + 8, 0u), cvt8<false>(y + 16, 0u),
                              cvt8<false>(y + 24, 0u)};
      const float L = loss_of_codes32<WMSE>(z, wg, kc, up);
      float Lm = ok ? L : __builtin_inff();
      int em = ok ? E : 0x7FFFFFFF;
      row_argmin16(Lm, em);
      const int es = em == 0x7FFFFFFF ? max(-127, eb + lo) : em;
      V = pow2f(es);
      R = pow2f(-es);
      if (live && t == 0) scales[(int64_t)r * (cols / 32) + ((i1 + 8 * tt) >> 5)] = (uint8_t)(es + 127);
    }
    if constexpr (!GIVEN && !MX && (tt & 1) == 0) {
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
        un0 = *reinterpret_cast<const f32x4 *>(&Ub[i + 1][8 * t]);
        un1 = *reinterpret_cast<const f32x4 *>(&Ub[i + 1][8 * t + 4]);
        rdn = rdiag[i + 1];
      }
      if constexpr (GIVEN) {  // this column's fixed scale, read one column ahead like its U row
        V = vgn;
        R = rgn;
        if (i + 1 < kGptqBatch) {
          vgn = Vg[tid >> 4][i + 1];
          rgn = Rg[tid >> 4][i + 1];
        }
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
// errors of kn already quantized columns: the near update (one batch of 128
// columns onto the rest of its block) as a dense contraction on fp32 MFMA
// (32x32x2).  With K = 128 it is short and latency-bound, where small tiles
// keep enough workgroups in flight.  A workgroup computes a 64 x 64 tile, each wave a
// 32 x 32 sub-tile whose 16 accumulator rows per lane are read from W at the
// start (their HBM latency then hides behind the contraction instead of
// stalling the epilogue).  E and U are staged through LDS in K chunks of 32:
// E row-major with a padded stride of 33 floats, U k-major, so the stores and
// the operand reads of each k step hit distinct banks.  The k steps run in
// ascending order, so every output element accumulates in the same order.
constexpr int kUpdKc = 32;

// C / ldc: where the output tile's current values are read (W, or the caller's weight for
// columns no update has touched yet); the result goes to W.
__global__ __launch_bounds__(kThreads) void gptq_update_kernel(float *W, int64_t ld, const float *C, int64_t ldc,
                                                               int rows, int cols, int i1, int kn, int cbeg,
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
    cur[v] = row < rows ? C[(int64_t)row * ldc + c0 + wc * 32 + lr] : 0.0f;
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

// The far update (a block's 1024 error columns against all later columns) on the bf16 matrix cores
// at fp32-class accuracy.  Every fp32 operand x is split exactly into three bf16 parts by round to
// nearest even, x = h + m + l: x - h and (x - h) - m are exact in fp32, |m| <= 2^-8 |x|,
// |l| <= 2^-16 |x|, and l fits bf16's 8-bit significand.  Of the nine part products the kernel keeps
// the six down to order 2^-16 (hh, hm, mh, hl, mm, lh); the three it drops (ml, lm, ll) add up to at
// most about 2^-23 |a b| per product, the size of an fp32 product's own rounding.  bf16 products are
// exact in the MFMA's fp32 accumulation, so the result matches an fp32 contraction to within fp32
// summation error, at six bf16 MFMAs (32x32x16) where fp32 needs eight (32x32x2) at a sixteenth of
// the rate.  A 128 x 128 workgroup tile; K in stages of 16 (one bf16 MFMA step).  Each stage's E
// and U values are split once as they go from registers into LDS: E row-major, U column-major, each
// part its own [128][KC] bf16 array, so an operand is one 16-byte read.  A row's 16-byte chunks are
// permuted by an XOR with bits of the row index, which puts 16 consecutive rows' reads of one chunk,
// and the stores, on distinct banks.  Finite operands below 2^127 (h must not round to infinity).
// K elements per stage: one bf16 MFMA step.  Stages of 32 (two steps per barrier) need 96 KB of LDS,
// one workgroup per CU, and measured slower.
constexpr int kSplitKc = 16;
// offset in bf16 of element k (0..KC-1) of row r in a staged part array of KC-element rows
template <int KC>
__device__ __forceinline__ int split_idx(int r, int k) {
  constexpr int NC = KC / 8, SH = NC == 2 ? 3 : 2;  // 16-byte chunks per row; row bits that permute them
  static_assert(NC == 2 || NC == 4, "16- or 32-element rows");
  return KC * r + 8 * ((k >> 3) ^ ((r >> SH) & (NC - 1))) + (k & 7);
}
constexpr int kSplitWaves = 8;  // measured faster than 4 waves (2 x 2 blocks each) at every far-update size
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// Two floats to their three bf16 parts, each pair packed low element first.
__device__ __forceinline__ void split_bf16x3(float x0, float x1, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x0, x1}), bf16x2v));
  const float r0 = x0 - as_f(h << 16), r1 = x1 - as_f(h & 0xFFFF0000u);
  m = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r0, r1}), bf16x2v));
  const float s0 = r0 - as_f(m << 16), s1 = r1 - as_f(m & 0xFFFF0000u);
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{s0, s1}), bf16x2v));
}

// NW waves per workgroup: 4 (each wave a 2 x 2 grid of 32 x 32 blocks) or 8 (each wave 1 x 2); KC K
// elements per stage (16 or 32).
template <int NW, int KC>
__global__ __launch_bounds__(64 * NW) void gptq_update_split_kernel(float *W, int64_t ld, const float *C,
                                                                    int64_t ldc, int rows, int cols, int i1, int kn,
                                                                    int cbeg, const float *__restrict__ U) {
  constexpr int BM = 128, BN = 128, NT = 64 * NW, KS = KC / 16;
  constexpr int WR = NW / 2, TI = 4 / WR, TJ = 2;  // wave grid WR x 2; blocks per wave TI x TJ
  constexpr int EPT = BM * KC / NT;                 // values per thread per operand per stage
  constexpr int NPC = EPT;                          // split pieces per stage (pairs of E, then of U)
  constexpr int NMF = 6 * TI * TJ * KS;             // MFMAs per wave per stage
  static_assert(NMF == 3 * NPC, "a piece after every third MFMA");
  static_assert(EPT == 4 || EPT % 8 == 0, "a thread's parts are stored as 8-byte or 16-byte chunks");
  // [stage buffer][0: E rows, 1: U columns][part h, m, l][row or column, k] (split_idx)
  __shared__ __attribute__((aligned(16))) uint16_t S[2][2][3][BM * KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * BM, c0 = cbeg + blockIdx.y * BN;
  const int wr = wave % WR, wc = wave / WR;
  const int lr = lane & 31, lk = lane >> 5;
  // a stage: thread t takes EPT consecutive k of E row t / (KC / EPT) and of U column t / (KC / EPT)
  const int ar = tid / (KC / EPT), ak = EPT * (tid % (KC / EPT));
  const int bc = ar, bk = ak;
  // rows past the end read row 0: a row of E only reaches the same row of the output, which is not
  // stored
  const float *asrc = W + (int64_t)(r0 + ar < rows ? r0 + ar : 0) * ld + i1 + ak;
  const float *bsrc = U + (int64_t)(i1 + bk) * cols + c0 + bc;
  // stage kc's raw values into a / b (kc is clamped by the caller, so every load is in bounds)
  auto fetch = [&](int kc, float (&a)[EPT], float (&b)[EPT]) {
#pragma unroll
    for (int h = 0; h < EPT / 4; ++h) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(asrc + kc + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) a[4 * h + k] = v[k];
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) b[k] = bsrc[(int64_t)(kc + k) * cols];
  };
  // split piece q of a stage (q < EPT / 2: E pair q, else U pair q - EPT / 2) into ph / pm / pl;
  // after the last pair of each operand its parts are stored to LDS buffer buf
  constexpr int NW2 = EPT / 2;
  uint32_t ph[NW2], pm[NW2], pl[NW2];
  auto store = [&](uint16_t *part, int rr, int kk, const uint32_t (&v)[NW2]) {
    if constexpr (NW2 == 2) {
      *reinterpret_cast<uint2 *>(part + split_idx<KC>(rr, kk)) = uint2{v[0], v[1]};
    } else {
#pragma unroll
      for (int h = 0; h < NW2 / 4; ++h)
        *reinterpret_cast<u32x4 *>(part + split_idx<KC>(rr, kk + 8 * h)) =
            u32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
    }
  };
  auto piece = [&](int q, int buf, const float (&a)[EPT], const float (&b)[EPT]) {
    const float *x = q < NW2 ? a : b;
    const int qq = q % NW2;
    split_bf16x3(x[2 * qq], x[2 * qq + 1], ph[qq], pm[qq], pl[qq]);
    if (qq == NW2 - 1) {
      const int o = q < NW2 ? 0 : 1, rr = o ? bc : ar, kk = o ? bk : ak;
      store(S[buf][o][0], rr, kk, ph);
      store(S[buf][o][1], rr, kk, pm);
      store(S[buf][o][2], rr, kk, pl);
    }
  };
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{0};
  // Software pipeline over stages of KC: while stage kc's MFMAs run from LDS buffer buf, stage
  // kc + KC (loaded one stage earlier into as / bs) is split into the other buffer, one piece after
  // every third MFMA, and stage kc + 2 KC loads into an / bn.  Past the end the loads repeat the last
  // stage and the split fills a buffer nobody reads.  Terms go small products first, each term
  // across the wave's blocks in turn, so consecutive MFMAs never share an accumulator.
  const int klast = kn - KC;
  auto stage = [&](int kc, int buf, const float (&as)[EPT], const float (&bs)[EPT], float (&an)[EPT],
                   float (&bn)[EPT]) {
    fetch(min(kc + 2 * KC, klast), an, bn);
    bf16x8v av[KS][TI][3], bv[KS][TJ][3];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
          av[ks][i][2 - p] = *reinterpret_cast<const bf16x8v *>(
              &S[buf][0][2 - p][split_idx<KC>(wr * 32 * TI + 32 * i + lr, 16 * ks + 8 * lk)]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bv[ks][j][p] = *reinterpret_cast<const bf16x8v *>(
              &S[buf][1][p][split_idx<KC>(wc * 64 + 32 * j + lr, 16 * ks + 8 * lk)]);
      }
    constexpr int PA[6] = {2, 1, 0, 1, 0, 0}, PB[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
    for (int g = 0; g < NMF; ++g) {
      const int ks = g / (6 * TI * TJ), t = (g / (TI * TJ)) % 6, i = (g / TJ) % TI, j = g % TJ;
      acc[i][j] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks][i][PA[t]], bv[ks][j][PB[t]], acc[i][j], 0, 0, 0);
      if (g % 3 == 2) piece(g / 3, buf ^ 1, as, bs);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };
  float a0[EPT], b0[EPT], a1[EPT], b1[EPT];
  fetch(0, a0, b0);
#pragma unroll
  for (int q = 0; q < NPC; ++q) piece(q, 0, a0, b0);
  fetch(min(KC, klast), a0, b0);
  __syncthreads();
  for (int kc = 0; kc < kn; kc += 2 * KC) {  // kn is a multiple of 2 KC
    stage(kc, 0, a0, b0, a1, b1);
    stage(kc + KC, 1, a1, b1, a0, b0);
  }
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // accumulator v of block (i, j) in lane l: row 32 i + 8*(v/4) + 4*(l/32) + v%4, column 32 j + l%32
        const int row = r0 + wr * 32 * TI + 32 * i + 8 * (v >> 2) + 4 * lk + (v & 3);
        const int64_t col = c0 + wc * 64 + 32 * j + lr;
        if (row < rows) W[(int64_t)row * ld + col] = C[(int64_t)row * ldc + col] - acc[i][j][v];
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
  const int64_t g0 = (int64_t)blockIdx.x * kThreads + 64 * wave_index();
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
  const int64_t g0 = (int64_t)blockIdx.x * kThreads + 64 * wave_index();
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

// ------------------------------------------------ GPTQ, static reordering ----
// "Bridging the Gap Between Promise and Performance for Microscaling FP4 Quantization", 2. Metodologia,
// MR-GPTQ component 2: GPTQ's column order is applied once, while quantizing, so inference shuffles
// nothing.  The columns are processed in the caller's order perm (slot j holds stored column perm[j]);
// the groups, their scales and the codes stay in the stored order.

// inv[perm[j]] = j for every slot j (entries of perm outside [0, cols) are reported and clamped).  The
// call's first kernel: it takes the status slot.
__global__ __launch_bounds__(kThreads) void perm_inverse_kernel(const int32_t *__restrict__ perm, int cols,
                                                                 int32_t *__restrict__ inv, Status status) {
  const int j = blockIdx.x * kThreads + threadIdx.x;
  uint32_t err = 0u;
  if (j < cols) {
    const int p = perm[j];
    if (p < 0 || p >= cols) err = FP4Q_DATA_BAD_PERM;
    inv[min(max(p, 0), cols - 1)] = j;
  }
  status.finish(err);
}

// The weight in processing order, w[r][j] = w_in[r][perm[j]]: one workgroup per row (a row's random
// reads then fill one XCD's L2 once; spread over the workgroups of several XCDs, each fetched the whole
// row), four slots per thread and step (cols is a multiple of 128).  Row 0 also checks that perm is a
// permutation: a repeated entry leaves a slot whose entry of inv names another slot.
__global__ __launch_bounds__(kThreads) void perm_gather_kernel(const float *__restrict__ w_in, int64_t ld_in,
                                                                const int32_t *__restrict__ perm,
                                                                const int32_t *__restrict__ inv, int rows, int cols,
                                                                float *__restrict__ w, int64_t ld,
                                                                uint32_t *__restrict__ status) {
  // four steps of four slots per pass, every load of a pass issued before its first store; steps past
  // the row's end read slot 0 and store nothing
  constexpr int kSteps = 4;
  uint32_t err = 0u;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const float *src = w_in + (int64_t)r * ld_in;
    for (int jb = 4 * (int)threadIdx.x; jb < cols; jb += 4 * kThreads * kSteps) {
      int pc[kSteps][4];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int j0 = jb + 4 * kThreads * u;
#pragma unroll
        for (int k = 0; k < 4; ++k) pc[u][k] = j0 < cols ? min(max(perm[j0 + k], 0), cols - 1) : 0;
      }
      f32x4 v[kSteps];
#pragma unroll
      for (int u = 0; u < kSteps; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[u][k] = src[pc[u][k]];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int j0 = jb + 4 * kThreads * u;
        if (j0 < cols) {
          *reinterpret_cast<f32x4 *>(w + (int64_t)r * ld + j0) = v[u];
          if (r == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (inv[pc[u][k]] != j0 + k) err = FP4Q_DATA_BAD_PERM;
          }
        }
      }
    }
  }
  if (err) atomicOr(status, err);
}

// Codes back in the stored order: the code of stored column c sits at slot inv[c] of the
// processing-order codes cp (both [rows][cols / 2], low nibble first).  Sixteen columns per thread.
__global__ __launch_bounds__(kThreads) void codes_unpermute_kernel(const uint8_t *__restrict__ cp,
                                                                    const int32_t *__restrict__ inv, int rows,
                                                                    int cols, uint8_t *__restrict__ codes) {
  const int q = cols / 16;
  const int64_t total = (int64_t)rows * q;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (int64_t)gridDim.x * kThreads) {
    const int r = (int)(g / q), c0 = (int)(g % q) * 16;
    const uint8_t *row = cp + (int64_t)r * (cols / 2);
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int sl = min(max(inv[c0 + k], 0), cols - 1);
      const uint32_t nib = (row[sl >> 1] >> (4 * (sl & 1))) & 0xFu;
      word[k >> 3] |= nib << (4 * (k & 7));
    }
    *reinterpret_cast<uint2 *>(codes + (int64_t)r * (cols / 2) + c0 / 2) = make_uint2(word[0], word[1]);
  }
}

// The GPTQ batches of either format: per 128-column batch the batch kernel,
// then the lazy updates.  Within a block of kGptqBlock columns they follow a
// binary tree: after batch t of the block, with m the lowest set bit of t + 1,
// the last m batches' errors go to the next m batches' columns (m = 1, 2, 1,
// 4, 1, 2, 1: every column still gets every earlier batch's errors before its
// own batch, with the same flops as updating the whole rest of the block
// after every batch, in fewer wide launches).  After the block's last batch,
// all later columns get the block's error columns as one contraction.
//
// GIVEN: static reordering (gptq_batch_kernel's GIVEN mode): the columns are processing slots of the
// order perm, every group's scale is already in `scales`, and codes go to the slots' positions.
template <int FMT, bool GIVEN = false>
static void gptq_batches(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in, int64_t ld_in,
                         const float *hinv_chol, const float *importance, float *global_scale,
                         const uint32_t *partials, int n_partials, int off_lo, int off_hi, uint8_t *codes,
                         uint8_t *scales, uint32_t *status_slot, bool first_kernel, hipStream_t s,
                         const int32_t *perm = nullptr) {
  const int gb = ceil_div(rows, kGptqRowsPerWg);
  // w holds columns [0, held); a launch reads the current values of later columns from w_in (the
  // caller's weight, untouched so far), so w needs no copy of it (w_in == w: in place)
  int held = 0;
  int pk = -1;  // start of the batch whose errors the next batch kernel applies to its own columns
  auto near = [&](int k0, int kn, int c0, int c1) {  // errors of columns [k0, k0 + kn) onto [c0, c1)
    for (int lo = c0; lo < c1;) {
      const bool old = lo < held;
      const int hi = old ? std::min(c1, held) : c1;
      hipLaunchKernelGGL(gptq_update_kernel, dim3(ceil_div(rows, 64), (hi - lo) / 64), dim3(kThreads), 0, s, w, ld,
                         old ? w : w_in, old ? ld : ld_in, (int)rows, (int)cols, k0, kn, lo, hinv_chol);
      lo = hi;
    }
    held = std::max(held, c1);
  };
  auto far = [&](int k0, int kn, int c0, int c1) {
    for (int lo = c0; lo < c1;) {
      const bool old = lo < held;
      const int hi = old ? std::min(c1, held) : c1;
      hipLaunchKernelGGL((gptq_update_split_kernel<kSplitWaves, kSplitKc>), dim3(ceil_div(rows, 128), (hi - lo) / 128),
                         dim3(64 * kSplitWaves), 0, s, w, ld, old ? w : w_in, old ? ld : ld_in, (int)rows,
                         (int)cols, k0, kn, lo, hinv_chol);
      lo = hi;
    }
    held = std::max(held, c1);
  };
  for (int i1 = 0; i1 < cols; i1 += kGptqBatch) {
    // the first batch kernel is the call's first kernel unless a max pass ran before it, whose
    // partials it then reduces to S
    const Status status{status_slot, first_kernel && i1 == 0};
    const uint32_t *part = i1 == 0 ? partials : nullptr;
    const bool old = i1 < held;
    const float *src = old ? w : w_in;
    const int64_t lds = old ? ld : ld_in;
    if constexpr (GIVEN)
      hipLaunchKernelGGL((gptq_batch_kernel<false, FMT, true>), dim3(gb), dim3(kGptqBatchThreads), 0, s, w, ld, src,
                         lds, pk, (int)rows, (int)cols, i1, hinv_chol, nullptr, global_scale, part, n_partials,
                         off_lo, off_hi, codes, scales, status, perm);
    else if (importance)
      hipLaunchKernelGGL((gptq_batch_kernel<true, FMT>), dim3(gb), dim3(kGptqBatchThreads), 0, s, w, ld, src, lds,
                         pk, (int)rows, (int)cols, i1, hinv_chol, importance, global_scale, part, n_partials,
                         off_lo, off_hi, codes, scales, status);
    else
      hipLaunchKernelGGL((gptq_batch_kernel<false, FMT>), dim3(gb), dim3(kGptqBatchThreads), 0, s, w, ld, src, lds,
                         pk, (int)rows, (int)cols, i1, hinv_chol, importance, global_scale, part, n_partials,
                         off_lo, off_hi, codes, scales, status);
    held = std::max(held, i1 + kGptqBatch);
    pk = -1;
    const int i2 = i1 + kGptqBatch;
    const int b0 = i1 / kGptqBlock * kGptqBlock, b1 = std::min((int)cols, b0 + kGptqBlock);
    // batch t of the block (m = the lowest set bit of t + 1): the last m batches' errors onto the
    // next m batches' columns; for m = 1 the next batch kernel applies them itself
    const int tb = (i1 - b0) / kGptqBatch, m = (tb + 1) & -(tb + 1);
    if (i2 < b1 && m == 1)
      pk = i1;
    else if (i2 < b1)
      near(i2 - m * kGptqBatch, m * kGptqBatch, i2, std::min(b1, i2 + m * kGptqBatch));
    else if (b1 < cols)  // the far update (cols - b1 is a multiple of the 128-column tile)
      far(b0, b1 - b0, b1, (int)cols);
  }
}

static AmaxOut amax_out(void *workspace, const float *imp, int imp_n, bool first = true) {
  char *b = (char *)workspace;
  return AmaxOut{(uint32_t *)(b + kWsPartials), (uint32_t *)(b + kWsStatus), imp, imp_n, first};
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

// fp4q_quantize_nvfp4 on explicit scratch: the call's status word and
// kAmaxGroups words for the max-pass partials (ws_ok: the caller's scratch
// passed its check, reported in the argument-check order of the C ABI).
static fp4q_status_t quantize_nvfp4_on(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                       const float *importance, int block, fp4q_loss_t loss, int off_lo, int off_hi,
                                       int hadamard_n, uint32_t flags, uint8_t *codes, uint8_t *scales,
                                       float *global_scale, float *block_loss, int8_t *offsets, bool ws_ok,
                                       uint32_t *status, uint32_t *partials, hipStream_t s) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && (!x || !codes || !scales))) return FP4Q_ERR_NULL;
  if (loss != FP4Q_MSE && loss != FP4Q_WMSE) return FP4Q_ERR_ARG;
  if (loss == FP4Q_WMSE && !importance && !empty) return FP4Q_ERR_NULL;
  if (!ws_ok) return FP4Q_ERR_WORKSPACE;
  if (block != 16) return FP4Q_ERR_SHAPE;
  if (off_lo > 0 || off_hi < 0 || off_lo < -126 || off_hi > 126) return FP4Q_ERR_ARG;
  if (flags & ~(FP4Q_GIVEN_SCALE | FP4Q_ACCUMULATE_STATUS)) return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, hadamard_n);
  if (st != FP4Q_OK) return st;
  const bool wmse = loss == FP4Q_WMSE;
  if (!empty && wmse && !aligned(importance, 16)) return FP4Q_ERR_ALIGN;
  if (!empty && (!aligned(codes, 8) || (block_loss && !aligned(block_loss, 4)))) return FP4Q_ERR_ALIGN;

  const bool given = flags & FP4Q_GIVEN_SCALE;
  const bool accumulate = flags & FP4Q_ACCUMULATE_STATUS;

  // The call's first kernel takes the status slot: the global-max pass, or with a given scale the sweep
  // (which then validates the scale and the importance itself).  A call that adds to the word does
  // not take it.  An empty tensor gets one small kernel for the slot and the scale.
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, !accumulate,
                       given ? global_scale : nullptr, given ? nullptr : global_scale);
    return last_hip_status();
  }

  const int cpr = (int)(cols / 16);
  const int n_partials =
      given ? 0
            : launch_amax(x, dtype, rows, cols, ld, hadamard_n,
                          AmaxOut{partials, status, wmse ? importance : nullptr, (int)cols, !accumulate}, s);

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
  a.partials = partials;
  a.n_partials = n_partials;
  a.given_scale = given ? global_scale : nullptr;
  a.check_inputs = given;
  a.status_first = given && !accumulate;
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

extern "C" fp4q_status_t fp4q_quantize_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                             int64_t ld, const float *importance, int block,
                                             fp4q_loss_t loss, int off_lo, int off_hi, int hadamard_n,
                                             uint32_t flags, uint8_t *codes, uint8_t *scales,
                                             float *global_scale, float *block_loss, int8_t *offsets,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  const bool ws_ok = workspace && workspace_bytes >= kWorkspaceBytes && aligned(workspace, 8);
  char *ws = (char *)workspace;  // offsets into it only once it is known to be there
  return quantize_nvfp4_on(x, dtype, rows, cols, ld, importance, block, loss, off_lo, off_hi, hadamard_n, flags,
                           codes, scales, global_scale, block_loss, offsets, ws_ok,
                           ws_ok ? (uint32_t *)(ws + kWsStatus) : nullptr,
                           ws_ok ? (uint32_t *)(ws + kWsPartials) : nullptr, (hipStream_t)stream);
}

// ------------------------------------------------ no-allocation variant ----
// Scratch of fp4q_quantize_nvfp4_noalloc: the global-max pass's
// per-workgroup partials (at most kAmaxGroups, whatever the tensor's size),
// in a device array of this library rather than a caller workspace.  Each
// GPU holds its own copy until the process ends; host code reaches a
// device's copy only through the address hipGetSymbolAddress gives on that
// device (the array's name is a host-side stand-in).
static __device__ __align__(256) uint32_t scratch[kAmaxGroups];

constexpr int kMaxDevices = 64;
static std::atomic<uint32_t *> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// This device's address of `scratch`, looked up once per device (with that
// device current, on its first call).
static fp4q_status_t scratch_of_current_device(uint32_t **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4Q_ERR_HIP;
  uint32_t *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return FP4Q_ERR_HIP;
      p = (uint32_t *)addr;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP4Q_OK;
}

extern "C" size_t fp4q_noalloc_scratch_bytes(void) { return sizeof(scratch); }

extern "C" fp4q_status_t fp4q_quantize_nvfp4_noalloc(const void *x, fp4q_dtype_t dtype, int64_t rows,
                                                     int64_t cols, int64_t ld, const float *importance, int block,
                                                     fp4q_loss_t loss, int off_lo, int off_hi, int hadamard_n,
                                                     uint32_t flags, uint8_t *codes, uint8_t *scales,
                                                     float *global_scale, float *block_loss, int8_t *offsets,
                                                     uint32_t *status, void *stream) {
  if (!status) return FP4Q_ERR_NULL;
  if (!aligned(status, 8)) return FP4Q_ERR_ALIGN;  // the status slot is one 64-bit word
  uint32_t *partials = nullptr;
  const fp4q_status_t st = scratch_of_current_device(&partials);
  if (st != FP4Q_OK) return st;
  // the max pass writes at most kAmaxGroups partials, the size of the array, for any input: no input
  // size exceeds the scratch
  static_assert(sizeof(scratch) >= kAmaxGroups * sizeof(uint32_t), "scratch holds every max-pass partial");
  return quantize_nvfp4_on(x, dtype, rows, cols, ld, importance, block, loss, off_lo, off_hi, hadamard_n, flags,
                           codes, scales, global_scale, block_loss, offsets, true, status, partials,
                           (hipStream_t)stream);
}

extern "C" fp4q_status_t fp4q_global_scale_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                                 int64_t ld, int hadamard_n, float *global_scale, void *workspace,
                                                 size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && !x)) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes || !aligned(workspace, 8)) return FP4Q_ERR_WORKSPACE;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, 16, hadamard_n);
  if (st != FP4Q_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, (uint32_t *)((char *)workspace + kWsStatus),
                       true, nullptr, global_scale);
    return last_hip_status();
  }
  // the max pass and the reduction of its partials, as at the start of fp4q_quantize_nvfp4
  const int n_partials = launch_amax(x, dtype, rows, cols, ld, hadamard_n, amax_out(workspace, nullptr, 0), s);
  hipLaunchKernelGGL(scale_from_partials_kernel, dim3(1), dim3(kThreads), 0, s,
                     (const uint32_t *)((const char *)workspace + kWsPartials), n_partials, global_scale,
                     (uint32_t *)((char *)workspace + kWsStatus));
  return last_hip_status();
}

// fp4q_quantize_mxfp4 on a checked workspace's status word; status_first: the sweep is the call's
// first kernel and takes the status slot (else it adds to the word).
static fp4q_status_t quantize_mxfp4_on(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                       const float *importance, int block, fp4q_loss_t loss, int off_lo,
                                       int off_hi, int hadamard_n, uint8_t *codes, uint8_t *scales,
                                       float *block_loss, int8_t *offsets, bool ws_ok, uint32_t *status,
                                       bool status_first, hipStream_t s) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!x || !codes || !scales)) return FP4Q_ERR_NULL;
  if (loss != FP4Q_MSE && loss != FP4Q_WMSE) return FP4Q_ERR_ARG;
  if (loss == FP4Q_WMSE && !importance && !empty) return FP4Q_ERR_NULL;
  if (!ws_ok) return FP4Q_ERR_WORKSPACE;
  if (block != 32) return FP4Q_ERR_SHAPE;
  if (off_lo > 0 || off_hi < 0 || off_lo < -16 || off_hi > 16) return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, hadamard_n);
  if (st != FP4Q_OK) return st;
  const bool wmse = loss == FP4Q_WMSE;
  if (!empty && wmse && !aligned(importance, 16)) return FP4Q_ERR_ALIGN;
  if (!empty && (!aligned(codes, 8) || (block_loss && !aligned(block_loss, 4)))) return FP4Q_ERR_ALIGN;

  // the sweep is the call's only kernel and takes the status slot; an empty call gets a small kernel for it
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, status_first, nullptr, nullptr);
    return last_hip_status();
  }

  const int bpr = (int)(cols / 32);  // one lane per 32-element block
  SweepArgs a;
  a.x = x;
  a.ld = ld;
  a.rows = (int)rows;
  a.cols = (int)cols;
  a.cpr = bpr;
  a.imp = wmse ? importance : nullptr;
  a.off_lo = off_lo;
  a.off_hi = off_hi;
  a.nbands = ceil_div(bpr, 64);
  a.rows_per_tile = pick_rows_per_tile((int)rows, a.nbands, kMxTileTarget);
  a.ntiles = a.nbands * ceil_div(rows, a.rows_per_tile);
  a.partials = nullptr;
  a.n_partials = 0;
  a.given_scale = nullptr;
  a.check_inputs = true;  // no max pass read the importance
  a.status_first = status_first;
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

extern "C" fp4q_status_t fp4q_quantize_mxfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                             int64_t ld, const float *importance, int block,
                                             fp4q_loss_t loss, int off_lo, int off_hi, int hadamard_n,
                                             uint8_t *codes, uint8_t *scales, float *block_loss,
                                             int8_t *offsets, void *workspace, size_t workspace_bytes,
                                             void *stream) {
  const bool ws_ok = workspace && workspace_bytes >= kWorkspaceBytes && aligned(workspace, 8);
  return quantize_mxfp4_on(x, dtype, rows, cols, ld, importance, block, loss, off_lo, off_hi, hadamard_n, codes,
                           scales, block_loss, offsets, ws_ok,
                           ws_ok ? (uint32_t *)((char *)workspace + kWsStatus) : nullptr, true,
                           (hipStream_t)stream);
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
  if (!workspace || workspace_bytes < kWorkspaceBytes || !aligned(workspace, 8)) return FP4Q_ERR_WORKSPACE;
  if (sub_block != 4 && sub_block != 8 && sub_block != 16 && !(sub_block == 32 && block == 32))
    return FP4Q_ERR_ARG;
  fp4q_status_t st = check_matrix(x, dtype, rows, cols, ld, block, 0);
  if (st != FP4Q_OK) return st;
  if (!empty &&
      (!aligned(codes, 8) || (dequant_out && !aligned(dequant_out, 16)) || (coeffs && !aligned(coeffs, 2))))
    return FP4Q_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  // the quantizer is the call's only kernel and takes the status slot; an empty call gets a small one
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, true, nullptr, nullptr);
    return last_hip_status();
  }
  const int cpr = (int)(cols / 16);
  const int total = (int)(rows * cpr);
  const int grid = ceil_div(total, kThreads);
  with_dtype(dtype, [&](auto tp) {
    using T = std::remove_const_t<std::remove_pointer_t<decltype(tp)>>;
    auto go = [&](auto fmt_c, auto sub_c) {
      constexpr int FM = decltype(fmt_c)::value, SB = decltype(sub_c)::value;
      hipLaunchKernelGGL((relaxed_quant_kernel<T, FM, SB>), dim3(grid), dim3(kThreads), 0, s, (const T *)x, ld,
                         cpr, (int)cols, total, scales, global_scale, coeffs, codes, dequant_out,
                         Status{status, true});
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

// The weight is read from w_in (ld_in), or from w when w_in is NULL; w is the working storage.
static bool gptq_source_ok(const float *w_in, int64_t ld_in, int64_t cols) {
  return !w_in || (ld_in >= cols);
}

extern "C" fp4q_status_t fp4q_gptq_nvfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                         int64_t ld_in, const float *hinv_chol, const float *importance,
                                         int off_lo, int off_hi, uint32_t flags, uint8_t *codes,
                                         uint8_t *scales, float *global_scale, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!global_scale || (!empty && (!w || !hinv_chol || !codes || !scales))) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes || !aligned(workspace, 8)) return FP4Q_ERR_WORKSPACE;
  if (off_lo > 0 || off_hi < 0 || off_hi - off_lo > 15) return FP4Q_ERR_ARG;
  if (flags & ~FP4Q_GIVEN_SCALE) return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols || cols % kGptqBatch || !gptq_source_ok(w_in, ld_in, cols))
    return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (!empty && (!aligned(w, 16) || ld % 4 || !aligned(hinv_chol, 16) || !aligned(codes, 4) ||
                 (importance && !aligned(importance, 4)) || (w_in && (!aligned(w_in, 16) || ld_in % 4))))
    return FP4Q_ERR_ALIGN;
  if (!w_in) w_in = w, ld_in = ld;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  const bool given = flags & FP4Q_GIVEN_SCALE;
  // the call's first kernel takes the status slot: the global-max pass, or with a given scale the first
  // batch kernel (which also validates the scale); an empty matrix gets a small kernel for it
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, true, given ? global_scale : nullptr,
                       given ? nullptr : global_scale);
    return last_hip_status();
  }
  // without a given scale, the max pass runs first and the first batch kernel reduces its partials
  const uint32_t *partials = given ? nullptr : (const uint32_t *)((char *)workspace + kWsPartials);
  const int n_partials =
      given ? 0 : launch_amax(w_in, FP4Q_F32, rows, cols, ld_in, 0, amax_out(workspace, nullptr, 0), s);
  gptq_batches<FP4Q_NVFP4>(w, rows, cols, ld, w_in, ld_in, hinv_chol, importance, global_scale, partials,
                           n_partials, off_lo, off_hi, codes, scales, status, given, s);
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_gptq_mxfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                         int64_t ld_in, const float *hinv_chol, const float *importance,
                                         int off_lo, int off_hi, uint8_t *codes, uint8_t *scales,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!w || !hinv_chol || !codes || !scales)) return FP4Q_ERR_NULL;
  if (!workspace || workspace_bytes < kWorkspaceBytes || !aligned(workspace, 8)) return FP4Q_ERR_WORKSPACE;
  if (off_lo > 0 || off_hi < 0 || off_hi - off_lo > 15) return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols || cols % kGptqBatch || !gptq_source_ok(w_in, ld_in, cols))
    return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (!empty && (!aligned(w, 16) || ld % 4 || !aligned(hinv_chol, 16) || !aligned(codes, 4) ||
                 (importance && !aligned(importance, 4)) || (w_in && (!aligned(w_in, 16) || ld_in % 4))))
    return FP4Q_ERR_ALIGN;
  if (!w_in) w_in = w, ld_in = ld;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  // the first batch kernel takes the status slot; an empty matrix gets a small kernel for it
  if (empty) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, true, nullptr, nullptr);
    return last_hip_status();
  }
  gptq_batches<FP4Q_MXFP4>(w, rows, cols, ld, w_in, ld_in, hinv_chol, importance, nullptr, nullptr, 0, off_lo,
                           off_hi, codes, scales, status, true, s);
  return last_hip_status();
}

// --------------------------------------------------- static reordering ----
// Workspace of the static-order GPTQ calls: the quantize workspace (status word, max-pass partials), then
// the inverse order (int32 per column), then the codes in processing order.
static int64_t round_up256(int64_t n) { return (n + 255) / 256 * 256; }
static int64_t static_ws_inv(void) { return (int64_t)kWorkspaceBytes; }
static int64_t static_ws_codes(int64_t cols) { return static_ws_inv() + round_up256(4 * cols); }

extern "C" size_t fp4q_gptq_static_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (size_t)(static_ws_codes(cols) + round_up256(rows * (cols / 2)));
}

// Argument checks of both static-order calls (the format's own window and alignment rules aside).
static fp4q_status_t check_gptq_static(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                       int64_t ld_in, const int32_t *perm, const float *hinv_chol,
                                       const float *importance, int off_lo, int off_hi, uint8_t *codes,
                                       uint8_t *scales, void *workspace, size_t workspace_bytes) {
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!w || !w_in || !perm || !hinv_chol || !codes || !scales)) return FP4Q_ERR_NULL;
  if (!workspace || !aligned(workspace, 256) ||
      (rows >= 0 && cols >= 0 && workspace_bytes < fp4q_gptq_static_workspace_bytes(rows, cols)))
    return FP4Q_ERR_WORKSPACE;
  if (off_lo > 0 || off_hi < 0 || off_hi - off_lo > 15) return FP4Q_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols || cols % kGptqBatch || ld_in < cols) return FP4Q_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (rows * (cols / 16) >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)))
    return FP4Q_ERR_SHAPE;
  if (!empty && (!aligned(w, 16) || ld % 4 || !aligned(w_in, 16) || ld_in % 4 || !aligned(hinv_chol, 16) ||
                 !aligned(codes, 8) || !aligned(perm, 4) || (importance && !aligned(importance, 16))))
    return FP4Q_ERR_ALIGN;
  if (!empty) {  // the weight is gathered into w, so the two must not share memory
    const uintptr_t a0 = (uintptr_t)w, a1 = a0 + (uintptr_t)(((rows - 1) * ld + cols) * 4);
    const uintptr_t b0 = (uintptr_t)w_in, b1 = b0 + (uintptr_t)(((rows - 1) * ld_in + cols) * 4);
    if (a0 < b1 && b0 < a1) return FP4Q_ERR_ARG;
  }
  return FP4Q_OK;
}

// The steps shared by both formats around the scale pass `scales_pass` (which must only add to the status
// word): the inverse order (the call's first kernel), the weight in processing order, the scales, the
// GPTQ batches with fixed scales, and the codes back to the stored order.
template <int FMT, typename ScalePass>
static fp4q_status_t gptq_static_run(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                     int64_t ld_in, const int32_t *perm, const float *hinv_chol, int off_lo,
                                     int off_hi, uint8_t *codes, uint8_t *scales, float *global_scale,
                                     void *workspace, hipStream_t s, ScalePass scales_pass) {
  char *ws = (char *)workspace;
  uint32_t *status = (uint32_t *)(ws + kWsStatus);
  int32_t *inv = (int32_t *)(ws + static_ws_inv());
  uint8_t *codes_p = (uint8_t *)(ws + static_ws_codes(cols));
  hipLaunchKernelGGL(perm_inverse_kernel, dim3(ceil_div(cols, kThreads)), dim3(kThreads), 0, s, perm, (int)cols,
                     inv, Status{status, true});
  hipLaunchKernelGGL(perm_gather_kernel, dim3((int)std::min<int64_t>(rows, 16384)), dim3(kThreads), 0, s, w_in,
                     ld_in, perm, inv, (int)rows, (int)cols, w, ld, status);
  const fp4q_status_t st = scales_pass();
  if (st != FP4Q_OK) return st;
  gptq_batches<FMT, true>(w, rows, cols, ld, w, ld, hinv_chol, nullptr, global_scale, nullptr, 0, off_lo, off_hi,
                          codes_p, scales, status, false, s, perm);
  const int64_t sixteens = rows * (cols / 16);
  hipLaunchKernelGGL(codes_unpermute_kernel,
                     dim3((int)std::min<int64_t>(ceil_div(sixteens, (int64_t)kThreads), 8192)), dim3(kThreads), 0,
                     s, codes_p, inv, (int)rows, (int)cols, codes);
  return last_hip_status();
}

extern "C" fp4q_status_t fp4q_gptq_static_nvfp4(float *w, int64_t rows, int64_t cols, int64_t ld,
                                                const float *w_in, int64_t ld_in, const int32_t *perm,
                                                const float *hinv_chol, const float *importance, int off_lo,
                                                int off_hi, uint32_t flags, uint8_t *codes, uint8_t *scales,
                                                float *global_scale, void *workspace, size_t workspace_bytes,
                                                void *stream) {
  if (!global_scale) return FP4Q_ERR_NULL;
  fp4q_status_t st = check_gptq_static(w, rows, cols, ld, w_in, ld_in, perm, hinv_chol, importance, off_lo, off_hi,
                                       codes, scales, workspace, workspace_bytes);
  if (st != FP4Q_OK) return st;
  if (flags & ~FP4Q_GIVEN_SCALE) return FP4Q_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  const bool given = flags & FP4Q_GIVEN_SCALE;
  if (rows == 0 || cols == 0) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, true, given ? global_scale : nullptr,
                       given ? nullptr : global_scale);
    return last_hip_status();
  }
  return gptq_static_run<FP4Q_NVFP4>(
      w, rows, cols, ld, w_in, ld_in, perm, hinv_chol, off_lo, off_hi, codes, scales, global_scale, workspace, s,
      [&]() {
        // S and every group's scale: the sweep on the stored weight (codes are overwritten later)
        return quantize_nvfp4_on(w_in, FP4Q_F32, rows, cols, ld_in, importance, 16,
                                 importance ? FP4Q_WMSE : FP4Q_MSE, off_lo, off_hi, 0,
                                 flags | FP4Q_ACCUMULATE_STATUS, codes, scales, global_scale, nullptr, nullptr, true,
                                 status, (uint32_t *)((char *)workspace + kWsPartials), s);
      });
}

extern "C" fp4q_status_t fp4q_gptq_static_mxfp4(float *w, int64_t rows, int64_t cols, int64_t ld,
                                                const float *w_in, int64_t ld_in, const int32_t *perm,
                                                const float *hinv_chol, const float *importance, int off_lo,
                                                int off_hi, uint8_t *codes, uint8_t *scales, void *workspace,
                                                size_t workspace_bytes, void *stream) {
  fp4q_status_t st = check_gptq_static(w, rows, cols, ld, w_in, ld_in, perm, hinv_chol, importance, off_lo, off_hi,
                                       codes, scales, workspace, workspace_bytes);
  if (st != FP4Q_OK) return st;
  if (off_lo < -16 || off_hi > 16) return FP4Q_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *status = (uint32_t *)((char *)workspace + kWsStatus);
  if (rows == 0 || cols == 0) {
    hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(64), 0, s, status, true, nullptr, nullptr);
    return last_hip_status();
  }
  return gptq_static_run<FP4Q_MXFP4>(
      w, rows, cols, ld, w_in, ld_in, perm, hinv_chol, off_lo, off_hi, codes, scales, nullptr, workspace, s, [&]() {
        return quantize_mxfp4_on(w_in, FP4Q_F32, rows, cols, ld_in, importance, 32,
                                 importance ? FP4Q_WMSE : FP4Q_MSE, off_lo, off_hi, 0, codes, scales, nullptr,
                                 nullptr, true, status, false, s);
      });
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
