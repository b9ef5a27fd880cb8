// Device code shared by the prefill, decode and plan kernels (gfx950).
//
// Window definitions follow "ATFlash — Per-RoPE-Wavelength Attention
// Windows", README "The idea": pair r of a score cell at distance delta is
// kept iff delta <= W_r (integer window W_r = floor(k * 2*pi / theta_r),
// clamped here to INT32_MAX, which leaves every comparison with a distance
// below 2^31 unchanged).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxPairs = 64;      // head_dim <= 128 on the GPU
constexpr int kWindowInf = 0x7fffffff;

// Kernel-argument view of the window: integer windows and turns per position.
struct WindowArgs {
  int32_t w[kMaxPairs];     // W_r clamped to INT32_MAX (INT32_MAX when off)
  double phi[kMaxPairs];    // theta_r / (2*pi)
};

// sin and cos of 2*pi*t for |t| <= 1/2 turn.  Quarter-turn reduction
// (exact: t - q/4 with q = rint(4t)), then the Taylor series of sin to a^9
// and cos to a^10 on |a| <= pi/4 (truncation below 2e-11), then the quadrant.
__device__ __forceinline__ void sincos_turns(float t, float* s, float* c) {
  const float q = __builtin_rintf(4.0f * t);
  const float r = __builtin_fmaf(q, -0.25f, t);
  const float a = r * 6.28318530717958648f;
  const float a2 = a * a;
  float sp = __builtin_fmaf(a2, 2.75573192239858907e-6f, -1.98412698412698413e-4f);
  sp = __builtin_fmaf(a2, sp, 8.33333333333333333e-3f);
  sp = __builtin_fmaf(a2, sp, -1.66666666666666667e-1f);
  sp = __builtin_fmaf(a2, sp, 1.0f);
  const float sa = a * sp;
  float cp = __builtin_fmaf(a2, -2.75573192239858907e-7f, 2.48015873015873016e-5f);
  cp = __builtin_fmaf(a2, cp, -1.38888888888888889e-3f);
  cp = __builtin_fmaf(a2, cp, 4.16666666666666667e-2f);
  cp = __builtin_fmaf(a2, cp, -0.5f);
  const float ca = __builtin_fmaf(a2, cp, 1.0f);
  const int qi = ((int)q) & 3;   // angle = a + qi * pi/2
  const float s0 = (qi & 1) ? ca : sa, c0 = (qi & 1) ? sa : ca;
  *s = (qi & 2) ? -s0 : s0;
  *c = ((qi + 1) & 2) ? -c0 : c0;
}

// Accurate sin/cos of the RoPE angle pos * theta_r: the phase in turns is
// formed and reduced to [-1/2, 1/2] in double, then sincos_turns.
__device__ __forceinline__ void rope_sincos(int64_t pos, double phi, float* s, float* c) {
  double t = (double)pos * phi;
  t -= __builtin_rint(t);
  sincos_turns((float)t, s, c);
}

// Number of pairs whose window is shorter than delta, computed by one wave:
// lane r holds W_r (lanes >= h hold INT32_MAX).  delta is wave-uniform.
__device__ __forceinline__ int wave_pairs_below(int w_lane, int64_t delta) {
  const int64_t d = delta > (int64_t)kWindowInf ? (int64_t)kWindowInf : delta;
  return __popcll(__ballot((int64_t)w_lane < d));
}

// Smallest / largest distance over the visible cells of query positions
// [n_lo, n_hi] x key positions [m_lo, m_hi], all below 2^30 (every difference
// fits in int32); false if no cell is visible.  The prefill kernels take their
// per-tile pair ranges from this; the plan kernel runs it for every tile.
__device__ __forceinline__ bool span32(int n_lo, int n_hi, int m_lo, int m_hi, bool causal,
                                       int* dmin, int* dmax) {
  if (n_hi < n_lo || m_hi < m_lo) return false;
  if (causal) {
    if (m_lo > n_hi) return false;
    *dmin = max(n_lo - m_hi, 0);
    *dmax = n_hi - m_lo;
  } else {
    *dmin = m_hi < n_lo ? n_lo - m_hi : (m_lo > n_hi ? m_lo - n_hi : 0);
    *dmax = max(abs(n_hi - m_lo), abs(n_lo - m_hi));
  }
  return true;
}

// First k-step (8 pairs each) that some cell at distances >= dmin needs: the
// pairs below wave_pairs_below(dmin) are pruned for every such cell.
__device__ __forceinline__ int first_kstep(int w_lane, int dmin) {
  return __popcll(__ballot(w_lane < dmin)) >> 3;
}

// Smallest / largest distance over the visible cells of rows [n_lo, n_hi] x
// keys [m_lo, m_hi] (positions, 64-bit).  false if no cell is visible.
__device__ __forceinline__ bool tile_distance_range(int64_t n_lo, int64_t n_hi, int64_t m_lo,
                                                    int64_t m_hi, bool causal, int64_t* dmin,
                                                    int64_t* dmax) {
  if (n_hi < n_lo || m_hi < m_lo) return false;
  if (causal) {
    if (m_lo > n_hi) return false;
    *dmin = n_lo - m_hi > 0 ? n_lo - m_hi : 0;
    *dmax = n_hi - m_lo;
  } else {
    if (m_hi < n_lo) *dmin = n_lo - m_hi;
    else if (m_lo > n_hi) *dmin = m_lo - n_hi;
    else *dmin = 0;
    const int64_t a = n_hi - m_lo, b = n_lo - m_hi;
    const int64_t aa = a < 0 ? -a : a, bb = b < 0 ? -b : b;
    *dmax = aa > bb ? aa : bb;
  }
  return true;
}

// Per-cell predicate of a partially windowed pair: the term of pair p is
// dropped at query position n, key position m iff the distance exceeds W_p.
__device__ __forceinline__ bool pair_dropped(int64_t n, int64_t m, int wp, bool causal) {
  int64_t d = n - m;
  if (!causal && d < 0) d = -d;
  return d > (int64_t)wp;
}

// Cells of a tile are addressed by their key offset ko from a base key
// position kbase (ko in [0, span)).  For the query at position npos and a
// partially windowed pair with window wp, the pair's term is dropped at the
// cell iff ko < *lo || ko > *hi.  (Causal: distance npos - m > wp; non-causal:
// |npos - m| > wp.)  Positions are below 2^30, so with wp <= 2^31 - 1 every
// difference taken on the selected branch fits in int32; thresholds saturate
// to [-1, span].
__device__ __forceinline__ void drop_bounds(int npos, int wp, int kbase, bool causal, int span,
                                            int* lo, int* hi) {
  const int d0 = npos - kbase;                 // key offset of the query position
  *lo = (wp > d0) ? -1 : min(d0 - wp, span);
  *hi = span;
  if (!causal) *hi = (wp >= span - d0) ? span : max(d0 + wp, -1);
}

// Visibility of the cell at key offset ko: hidden iff ko > *fut (a key after
// the query, causal) or ko >= *end (past the last key n_end - 1).
__device__ __forceinline__ void hide_bounds(int npos, int kbase, int n_end, bool causal, int span,
                                            int* fut, int* end) {
  *fut = causal ? max(-1, min(npos - kbase, span)) : span;
  *end = max(0, min(n_end - kbase, span));
}

// Both lanes l and l^32 get f(x_l, x_{l^32}) for a symmetric f: the swap puts
// the other half's value beside each lane's own.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes of a stream that is read once (KV cache during decode): a
// non-temporal load, which keeps the stream from displacing reused lines in the
// caches and streams markedly faster from HBM on this GPU than an ordinary
// load.
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (round to nearest even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Round two floats to fp16 (round to nearest even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed pair of fp16 values (v_dot2_f32_f16 with ones).
__device__ __forceinline__ float sum_f16x2(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// Power-of-two range exponents for the fp16 matrix-core operands.  fp16
// keeps 3 more mantissa bits than bf16 but stops at 65504; a tensor whose
// largest magnitude M reaches 2^14 is stored as x * 2^-e with the smallest
// e >= 0 that brings M * 2^-e below 2^14 (rotated keys stay below 2^14.5),
// and 2^e is applied back exactly in fp32.  For inputs below 2^14 e = 0 and
// the operands are plain fp16 roundings.
__device__ __forceinline__ int range_exp_of_float(float m) {
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;
  return ex > 13 ? ex - 13 : 0;
}
// Same, from the magnitude bits (sign cleared) of a bf16 value.
__device__ __forceinline__ int range_exp_of_bf16(uint32_t mag) {
  const int ex = (int)((mag >> 7) & 0xff) - 127;
  return ex > 13 ? ex - 13 : 0;
}
// Largest bf16 magnitude (as bits) among the 8 values of a 16-byte chunk.
__device__ __forceinline__ uint32_t max_mag_bf16x8(u32x4 w, uint32_t acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = max(acc, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return acc;
}

// acc + lo + hi of a packed pair of bf16 values (v_dot2_f32_bf16 with ones).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

}  // namespace atw
