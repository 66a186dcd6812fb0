// Device helpers for the fp4q kernels (gfx950, wave64).
//
// Number formats (see include/fp4q.h for the page citations):
//   E2M1  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (code index 0..7)
//   E4M3  FP8 block scale, bias 7, 3 mantissa bits, 0x7E = 448 largest
//   E8M0  power-of-two block scale 2^(b - 127)
// Every helper here is exact or a single correctly rounded float32 step;
// the file is compiled with -ffp-contract=off so nothing is fused unless it
// is written as an explicit fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

constexpr int kLaneElems = 16;  // every lane owns 16 contiguous elements of a row
constexpr int kWaveLanes = 64;
constexpr int kWaves = 4;       // waves per workgroup
constexpr int kThreads = kWaveLanes * kWaves;
constexpr int kAmaxGroups = 256;  // max workgroups of the global-max pass

// Workspace layout (bytes): [0,4) status word, [256, 256 + 4*kAmaxGroups)
// per-workgroup maxima of |x| as float32 bit patterns.
constexpr size_t kWsStatus = 0;
constexpr size_t kWsPartials = 256;
constexpr size_t kWorkspaceBytes = 8192;
static_assert(kWsPartials + 4 * kAmaxGroups <= kWorkspaceBytes, "workspace layout");

__device__ __forceinline__ float as_f(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ------------------------------------------------------------ loads ----
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw 16-element chunk as loaded (16-byte aligned); the input is streamed
// once, so the loads are marked non-temporal.
template <typename T>
struct Raw;
template <>
struct Raw<uint16_t> {
  u32x4 v[2];
};
template <>
struct Raw<float> {
  f32x4 v[4];
};

__device__ __forceinline__ void load_raw(const uint16_t *p, Raw<uint16_t> &r) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
  r.v[0] = __builtin_nontemporal_load(q);
  r.v[1] = __builtin_nontemporal_load(q + 1);
}
__device__ __forceinline__ void load_raw(const float *p, Raw<float> &r) {
  const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) r.v[k] = __builtin_nontemporal_load(q + k);
}
__device__ __forceinline__ void widen(const Raw<uint16_t> &r, float z[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t w = r.v[k >> 2][k & 3];
    z[2 * k] = as_f(w << 16);
    z[2 * k + 1] = as_f(w & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen(const Raw<float> &r, float z[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) z[k] = r.v[k >> 2][k & 3];
}

// 16 consecutive elements starting at p widened to fp32.
template <typename T>
__device__ __forceinline__ void load16(const T *p, float z[16]) {
  Raw<T> r;
  load_raw(p, r);
  widen(r, z);
}

// ------------------------------------------------ wide row stores ----
// Flat chunk g0 + lane of a matrix with cpr chunks per row: row r and
// chunk c, from a wave-uniform g0 (a multiple of 64) with one scalar
// division per wave.  Returns false for lanes past total.
__device__ __forceinline__ bool lane_chunk(int64_t g0, int lane, int cpr, int64_t total, int &r, int &c) {
  const int64_t r0 = g0 / cpr;
  int cc = (int)(g0 - r0 * cpr) + lane;
  int rr = (int)r0;
  if (cpr >= 64) {
    const bool wrap = cc >= cpr;
    rr += wrap;
    cc -= wrap ? cpr : 0;
  } else {
    const int q = cc / cpr;
    rr += q;
    cc -= q * cpr;
  }
  r = rr;
  c = cc;
  return g0 + lane < total;
}

// Per-wave LDS staging for wave_store: NQ 16-byte quads per lane plus one
// quad of padding per 16 (bank spread).
template <int NQ>
struct WaveStage {
  u32x4 q[64 * NQ + 4 * NQ];
};

// Stores lane l's NQ quads to dst[NQ l .. NQ l + NQ) for all 64 lanes of a
// wave, whose outputs form one contiguous run of 64 NQ quads.  One lane per
// chunk would write 16 bytes every 16 NQ bytes per instruction; going
// through LDS, each store instruction writes 1 KB contiguously, and the
// stores are marked non-temporal (the output is not read again here).
// Every lane of the wave must take part.
template <int NQ>
__device__ __forceinline__ void wave_store(u32x4 *dst, const u32x4 (&v)[NQ], int lane, WaveStage<NQ> &st) {
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int j = NQ * lane + k;
    st.q[j + (j >> 4)] = v[k];
  }
  // lanes read what other lanes of the same wave wrote: LDS operations of a wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int j = 64 * k + lane;
    __builtin_nontemporal_store(st.q[j + (j >> 4)], dst + j);
  }
}

// ------------------------------------------------- cross-lane moves ----
// Value held by lane (lane ^ M) of the wave, M in {1, 2, 4}.
// Value of lane (l & ~15) + N, i.e. lane N of the caller's 16-lane DPP row
// (row_newbcast, CDNA3 and later).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(N >= 0 && N < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// One step of row_argmin16: combine with the lane that DPP control CTRL selects.
template <int CTRL>
__device__ __forceinline__ void argmin_step(float &L, int &p) {
  const float L2 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(L), CTRL, 0xF, 0xF, false));
  const int p2 = __builtin_amdgcn_mov_dpp(p, CTRL, 0xF, 0xF, false);
  const bool take = (L2 < L) | ((L2 == L) & (p2 < p));
  L = take ? L2 : L;
  p = take ? p2 : p;
}

// (loss, candidate) minimum over the 16 lanes of the caller's DPP row, ties
// to the smaller candidate, in every lane of the row: pairs (quad_perm
// [1,0,3,2]), quads ([2,3,0,1]), halves (row_half_mirror), the row
// (row_mirror).
__device__ __forceinline__ void row_argmin16(float &L, int &p) {
  argmin_step<0xB1>(L, p);
  argmin_step<0x4E>(L, p);
  argmin_step<0x141>(L, p);
  argmin_step<0x140>(L, p);
}

template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  int i = __float_as_int(v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else {
    static_assert(M == 4, "xor distance");
    r = __builtin_amdgcn_ds_swizzle(i, 0x101F);  // bitmask mode: and 0x1F, xor 4
  }
  return __int_as_float(r);
}

// Index of the caller's wave in its workgroup, as a wave-uniform (scalar)
// value: tile arithmetic and row loops derived from it run on the scalar unit.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Maximum of v over the 64 lanes of the wave, in every lane, by DPP (no LDS
// round trips): row shifts by 1, 2, 4 and 8 leave each 16-lane row's maximum
// in its lane 15 (lanes shifted in from outside a row read 0, the identity),
// row_bcast:15 and row_bcast:31 carry rows 0-1 and 0-2 upwards, so lane 63
// ends with the wave's maximum, which is read back as a scalar.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
  return v > o ? v : o;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0x111, 0xF>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xF>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xF>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xF>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ------------------------------------------------- block Hadamard ----
// fp32(1/sqrt(N)): 1/sqrt(2) rounds to 0x3F3504F3; the odd powers of two
// below are that value scaled by exact powers of two.
template <int N>
__device__ __forceinline__ float hadamard_scale() {
  if constexpr (N == 16) return 0.25f;
  else if constexpr (N == 32) return as_f(0x3E3504F3u);
  else if constexpr (N == 64) return 0.125f;
  else {
    static_assert(N == 128, "Hadamard size");
    return as_f(0x3DB504F3u);
  }
}

// Sylvester block Hadamard of the N-group this lane's 16 elements belong to
// (N/16 consecutive lanes hold one group).  Stages h = 1 .. N/2 in order;
// h < 16 stay inside the lane, h >= 16 pair lane l with lane l ^ (h/16).
template <int N>
__device__ __forceinline__ void fwht(float z[16], int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        float a = z[i], b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
  if constexpr (N >= 32) {
    const bool hi = lane & 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float o = xor_lane<1>(z[i]);
      z[i] = hi ? (o - z[i]) : (z[i] + o);
    }
  }
  if constexpr (N >= 64) {
    const bool hi = lane & 2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float o = xor_lane<2>(z[i]);
      z[i] = hi ? (o - z[i]) : (z[i] + o);
    }
  }
  if constexpr (N >= 128) {
    const bool hi = lane & 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float o = xor_lane<4>(z[i]);
      z[i] = hi ? (o - z[i]) : (z[i] + o);
    }
  }
  const float c = hadamard_scale<N>();
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = z[i] * c;
}

// ------------------------------------------------------------ E2M1 ----
// gfx950 packed FP4 conversions with a unit scale: nearest E2M1 value,
// ties to the even code, saturation at 6 (Inf included), the sign of -0.0
// kept, the first operand in the low nibble of the selected byte.  This
// matches the E2M1 definition on every float32 in [0, 16) (checked against
// an independent software rounding on the GPU).
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Writes the codes of (y0, y1) into byte BYTE of old (other bytes kept).
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, BYTE);
}

// The two E2M1 values (signed) held by byte BYTE of pk.
template <int BYTE>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t pk) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, BYTE);
}

// Codes of 8 values y[0..8) packed into one dword (element 2k in the low
// nibble of byte k).
__device__ __forceinline__ uint32_t cvt_fp4x8(const float y[8]) {
  uint32_t pk = 0;
  pk = cvt_fp4x2<0>(pk, y[0], y[1]);
  pk = cvt_fp4x2<1>(pk, y[2], y[3]);
  pk = cvt_fp4x2<2>(pk, y[4], y[5]);
  pk = cvt_fp4x2<3>(pk, y[6], y[7]);
  return pk;
}

// E2M1 values of the 8 codes in pk.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t pk, float q[8]) {
  const f32x2 a = fp4x2_to_f32<0>(pk), b = fp4x2_to_f32<1>(pk);
  const f32x2 c = fp4x2_to_f32<2>(pk), d = fp4x2_to_f32<3>(pk);
  q[0] = a.x; q[1] = a.y; q[2] = b.x; q[3] = b.y;
  q[4] = c.x; q[5] = c.y; q[6] = d.x; q[7] = d.y;
}

// ------------------------------------------------------------ E4M3 ----
// Value of a non-negative E4M3 pattern p in 1..126 (exact).
__device__ __forceinline__ float e4m3_value(int p) {
  if (p < 8) return (float)p * 0.001953125f;  // subnormal p * 2^-9
  return as_f(((uint32_t)((p >> 3) + 120) << 23) | ((uint32_t)(p & 7) << 20));
}

// Nearest non-negative E4M3 pattern to t >= 0, ties to the even pattern,
// saturating at 0x7E (448).
__device__ __forceinline__ int e4m3_rne_sat(float t) {
  if (!(t < 448.0f)) return 126;
  if (t < 0.015625f) return (int)rintf(t * 512.0f);  // subnormal grid m * 2^-9
  uint32_t b = as_u(t);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  const int e = (int)(b >> 23) - 127;
  const int m = (int)((b >> 20) & 7u);
  const int p = ((e + 7) << 3) | m;
  return p < 126 ? p : 126;
}

// ------------------------------------------------------------ E8M0 ----
// 2^e for e in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float pow2f(int e) {
  return e >= -126 ? as_f((uint32_t)(e + 127) << 23) : as_f(0x00400000u);
}

// Least E with 6 * 2^E >= a (a >= 0), clamped to [-127, 127].  With
// a = 1.f * 2^k (normal), 6 * 2^E >= a iff E >= k - 1 - [1.f <= 1.5].
__device__ __forceinline__ int mx_base_exponent(float a) {
  const uint32_t b = as_u(a);
  const int ef = (int)(b >> 23);
  if (ef == 0) return -127;  // zero or subnormal: 6 * 2^-127 covers it
  const int E = (ef - 127) - ((b & 0x7FFFFFu) <= 0x400000u ? 3 : 2) + 1;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

}  // namespace fp4q
