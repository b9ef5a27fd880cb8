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

// Accurate sin/cos of the RoPE angle pos * theta_r: the phase in turns is
// formed and reduced to [-1/2, 1/2] in double, then sincosf on |angle| <= pi.
__device__ __forceinline__ void rope_sincos(int64_t pos, double phi, float* s, float* c) {
  double t = (double)pos * phi;
  t -= __builtin_rint(t);
  const float a = (float)(t * 6.283185307179586);
  sincosf(a, s, c);
}

// Number of pairs whose window is shorter than delta, computed by one wave:
// lane r holds W_r (lanes >= h hold INT32_MAX).  delta is wave-uniform.
__device__ __forceinline__ int wave_pairs_below(int w_lane, int64_t delta) {
  const int64_t d = delta > (int64_t)kWindowInf ? (int64_t)kWindowInf : delta;
  return __popcll(__ballot((int64_t)w_lane < d));
}

// Smallest / largest distance over the visible cells of rows [n_lo, n_hi] x
// keys [m_lo, m_hi] (positions).  false if no cell is visible.
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
// |npos - m| > wp.)  Thresholds are clamped to [-1, span].
__device__ __forceinline__ void drop_bounds(int64_t npos, int wp, int64_t kbase, bool causal,
                                            int span, int* lo, int* hi) {
  const int64_t l = npos - (int64_t)wp - kbase;
  *lo = (int)max((int64_t)-1, min(l, (int64_t)span));
  *hi = span;
  if (!causal) {
    const int64_t h = npos + (int64_t)wp - kbase;
    *hi = (int)max((int64_t)-1, min(h, (int64_t)span));
  }
}

// Visibility of the cell at key offset ko: hidden iff ko > *fut (a key after
// the query, causal) or ko >= *end (past the last key n_end - 1).
__device__ __forceinline__ void hide_bounds(int64_t npos, int64_t kbase, int64_t n_end, bool causal,
                                            int span, int* fut, int* end) {
  const int64_t c = causal ? npos - kbase : (int64_t)span;
  *fut = (int)max((int64_t)-1, min(c, (int64_t)span));
  *end = (int)max((int64_t)0, min(n_end - kbase, (int64_t)span));
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

// acc + lo + hi of a packed pair of bf16 values (v_dot2_f32_bf16 with ones).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

}  // namespace atw
