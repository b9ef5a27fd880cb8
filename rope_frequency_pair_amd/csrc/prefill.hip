// Windowed causal prefill for gfx950 (MI355X).
//
// Method: "ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
// idea" and "Porting to something else": the window is a slice of the
// query-key contraction axis.  For a key tile, the pairs whose window is
// shorter than the tile's smallest query-key distance are never needed, so
// that prefix of the pre-RoPE key rows is never loaded; RoPE is applied to
// the rest as it is loaded and only the surviving pair slice is written to
// LDS.  The online softmax (running max, normalizer) is the ordinary one.
//
// Layout of the work (designed for CDNA4, not taken from the pages):
//  * one workgroup = 8 waves = 256 consecutive query rows of one query head;
//    a wave owns 32 rows; key tiles of 64 keys, double-buffered in LDS;
//  * scores are computed transposed, S^T = K' Q'^T, with
//    v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2f32), so each
//    lane holds 16 keys of one query column and the row max / sum are mostly
//    in-lane; lanes l and l+32 share a query;
//  * the contraction axis is ordered pair by pair ((r, r+h) adjacent,
//    "frequency-ordered"): one bf16 k-step of 16 covers 8 whole pairs, so the
//    retained pairs [r, h) are a contiguous range of k-steps;
//  * pairs that are in the window for some cells of a wave's tile and not for
//    others ("partial" pairs) are added first, one pair per MFMA, and after
//    each such pair the cells beyond its window are reset to zero; because
//    windows grow with r, this leaves exactly the kept partial terms; the
//    fully kept pairs are added after;
//  * O^T += V^T P^T with P^T taken straight from the S^T registers; V is
//    transposed into LDS (keys contiguous per head-dim row, in the key order
//    the S^T register layout produces);
//  * lazy rescaling of the output when the running max grows by more than
//    2^8 (the softmax result is unchanged, only fewer rescales).
#include "device_common.h"
#include "kernels.h"

namespace atw {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsW = 32;
constexpr int kTK = kPrefillTileK;
constexpr int kReanchor = 16;        // exact RoPE angles every 16 key tiles
constexpr float kRescaleLog2 = 8.0f;

template <typename T, int D>
struct Cfg {
  static constexpr int H = D / 2;
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int EPC = 16 / (int)sizeof(T);            // elements per 16-byte chunk
  static constexpr int NCH = H / EPC;                         // chunks per half row
  static constexpr int NK_TASKS = kTK * NCH;                  // K staging tasks per tile
  static constexpr int KT = (NK_TASKS + kThreads - 1) / kThreads;
  static constexpr int NV_TASKS = kBf16 ? 32 * (D / 8) : kTK * (D / 4);
  static constexpr int VT = (NV_TASKS + kThreads - 1) / kThreads;
  static constexpr int KROW = D + 16 / (int)sizeof(T);        // K' row (elements), 16 B pad
  static constexpr int VROWS = kBf16 ? D : kTK;               // bf16: V^T rows; fp32: V rows
  static constexpr int VROW = kBf16 ? (kTK + 8) : (D + 4);
  static constexpr int NKS = kBf16 ? D / 16 : H;              // QK^T k-steps
  static constexpr int ND = D / 32;                           // 32-wide head-dim blocks
};

template <typename T, int D>
struct Smem {
  T k[2][kTK][Cfg<T, D>::KROW];
  T v[2][Cfg<T, D>::VROWS][Cfg<T, D>::VROW];
  float2 step[D / 2];
};

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Key offset (within a 32-key block) of accumulator register v in lane half s
// for the 32x32 MFMA output layout.
__device__ __forceinline__ constexpr int acc_row(int v) { return 8 * (v >> 2) + (v & 3); }

template <typename T>
__device__ __forceinline__ u32x4 load16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillParams p) {
  using C = Cfg<T, D>;
  constexpr int H = C::H;
  constexpr int EPC = C::EPC;
  __shared__ Smem<T, D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sh = lane >> 5, l32 = lane & 31;

  // ---- work item: largest causal blocks first
  const int per_qb = p.h_q * p.batch;
  const int qb = p.n_qblk - 1 - (int)(blockIdx.x / per_qb);
  const int rem = (int)(blockIdx.x % per_qb);
  const int hq = rem % p.h_q, bb = rem / p.h_q;
  const int kvh = p.kvh[hq];

  const T* qbase = (const T*)p.q + bb * p.qs[0] + hq * p.qs[1];
  const T* kbase = (const T*)p.k + bb * p.ks[0] + kvh * p.ks[1];
  const T* vbase = (const T*)p.v + bb * p.vs[0] + kvh * p.vs[1];
  T* obase = (T*)p.o + bb * p.os[0] + hq * p.os[1];

  const bool causal = p.causal != 0;
  const int i0 = qb * kPrefillBlockRows;
  const int g_last = min(i0 + kPrefillBlockRows - 1, p.n_q - 1);
  const int w_first = i0 + wave * kRowsW;
  const int w_last = min(w_first + kRowsW - 1, p.n_q - 1);
  const bool wave_rows = w_first <= w_last;
  const int64_t n_lo = (int64_t)p.q_pos0 + w_first, n_hi = (int64_t)p.q_pos0 + w_last;
  const int64_t gn_lo = (int64_t)p.q_pos0 + i0, gn_hi = (int64_t)p.q_pos0 + g_last;
  const int qrow = min(w_first + l32, p.n_q - 1);
  const int64_t npos = (int64_t)p.q_pos0 + qrow;
  const int w_lane = lane < H ? p.win.w[lane] : kWindowInf;

  if (tid < H) {
    float s, c;
    rope_sincos(kTK, p.win.phi[tid], &s, &c);
    sm.step[tid] = make_float2(c, s);
  }

  // ---- query: load, rotate at its position, keep as MFMA operand
  const T* qrow_ptr = qbase + (int64_t)qrow * p.qs[2];
  bf16x8 qop[C::kBf16 ? C::NKS : 1];
  float qf[C::kBf16 ? 1 : H];
  if constexpr (C::kBf16) {
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int r0 = 8 * ks + 4 * sh;
      const u32x2 a = *reinterpret_cast<const u32x2*>(qrow_ptr + r0);
      const u32x2 b = *reinterpret_cast<const u32x2*>(qrow_ptr + H + r0);
      u32x4 packed;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x1 = (u & 1) ? bf16_hi(a[u >> 1]) : bf16_lo(a[u >> 1]);
        const float x2 = (u & 1) ? bf16_hi(b[u >> 1]) : bf16_lo(b[u >> 1]);
        float s, c;
        rope_sincos(npos, p.win.phi[r0 + u], &s, &c);
        packed[u] = pack_bf16(x1 * c - x2 * s, x2 * c + x1 * s);
      }
      qop[ks] = __builtin_bit_cast(bf16x8, packed);
    }
  } else {
#pragma unroll
    for (int r = 0; r < H; ++r) {
      const float x1 = (float)qrow_ptr[r], x2 = (float)qrow_ptr[H + r];
      float s, c;
      rope_sincos(npos, p.win.phi[r], &s, &c);
      qf[r] = sh ? (x2 * c + x1 * s) : (x1 * c - x2 * s);
    }
  }

  f32x16 oacc[C::ND];
#pragma unroll
  for (int b = 0; b < C::ND; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t kv_end = causal ? min((int64_t)p.n_kv, gn_hi + 1) : (int64_t)p.n_kv;
  const int n_kt = (int)((kv_end + kTK - 1) / kTK);

  // ---- staging tasks of this thread (fixed over tiles)
  int kj[C::KT], kc[C::KT];
  bool kon[C::KT];
#pragma unroll
  for (int i = 0; i < C::KT; ++i) {
    const int task = tid + i * kThreads;
    kon[i] = task < C::NK_TASKS;
    kj[i] = kon[i] ? task / C::NCH : 0;
    kc[i] = kon[i] ? task % C::NCH : 0;
  }
  int vtask[C::VT];
  bool von[C::VT];
#pragma unroll
  for (int i = 0; i < C::VT; ++i) {
    // when there are fewer V tasks than threads, give them to the threads
    // with the fewest K tasks (the last ones)
    const int t = C::NV_TASKS < kThreads ? (tid + kThreads - C::NV_TASKS) % kThreads : tid;
    vtask[i] = t + i * kThreads;
    von[i] = vtask[i] < C::NV_TASKS;
  }
  float rc[C::KT][EPC], rs[C::KT][EPC];   // cos/sin at the next staged tile
  u32x4 kreg[C::KT][2];
  u32x4 vreg[C::VT][C::kBf16 ? 2 : 1];

  // WG-wide first pair needed in tile t (the staging start)
  auto stage_lo = [&](int t) -> int {
    const int64_t m_lo = (int64_t)t * kTK;
    const int64_t m_hi = min(m_lo + kTK - 1, (int64_t)p.n_kv - 1);
    int64_t dmin = 0, dmax = 0;
    if (!tile_distance_range(gn_lo, gn_hi, m_lo, m_hi, causal, &dmin, &dmax)) return H;
    const int r = wave_pairs_below(w_lane, dmin);
    return C::kBf16 ? (r & ~7) : r;
  };

  auto stage_load = [&](int t, int rlo) {
#pragma unroll
    for (int i = 0; i < C::KT; ++i) {
      const int64_t m = (int64_t)t * kTK + kj[i];
      const bool need = kon[i] && (kc[i] + 1) * EPC > rlo && m < p.n_kv;
      if (need) {
        const T* src = kbase + m * p.ks[2] + kc[i] * EPC;
        kreg[i][0] = load16(src);
        kreg[i][1] = load16(src + H);
      } else {
        kreg[i][0] = u32x4{0, 0, 0, 0};
        kreg[i][1] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < C::VT; ++i) {
      if constexpr (C::kBf16) {
        const int pr = vtask[i] / (D / 8), dc = vtask[i] % (D / 8);
        const int64_t m = (int64_t)t * kTK + 2 * pr;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if (von[i] && m + e < p.n_kv)
            vreg[i][e] = load16(vbase + (m + e) * p.vs[2] + dc * 8);
          else
            vreg[i][e] = u32x4{0, 0, 0, 0};
        }
      } else {
        const int j = vtask[i] / (D / 4), dc = vtask[i] % (D / 4);
        const int64_t m = (int64_t)t * kTK + j;
        if (von[i] && m < p.n_kv)
          vreg[i][0] = load16(vbase + m * p.vs[2] + dc * 4);
        else
          vreg[i][0] = u32x4{0, 0, 0, 0};
      }
    }
  };

  auto stage_store = [&](int t, int buf, int rlo) {
#pragma unroll
    for (int i = 0; i < C::KT; ++i) {
      if (!kon[i]) continue;
      const int64_t m = (int64_t)t * kTK + kj[i];
      if (t % kReanchor == 0) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) rope_sincos(m, p.win.phi[kc[i] * EPC + e], &rs[i][e], &rc[i][e]);
      }
      if ((kc[i] + 1) * EPC > rlo) {
        T* dst = &sm.k[buf][kj[i]][2 * kc[i] * EPC];
        if constexpr (C::kBf16) {
          u32x4 o0, o1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wa = kreg[i][0][e >> 1], wb = kreg[i][1][e >> 1];
            const float x1 = (e & 1) ? bf16_hi(wa) : bf16_lo(wa);
            const float x2 = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
            const uint32_t pk = pack_bf16(x1 * rc[i][e] - x2 * rs[i][e], x2 * rc[i][e] + x1 * rs[i][e]);
            if (e < 4) o0[e] = pk; else o1[e - 4] = pk;
          }
          reinterpret_cast<u32x4*>(dst)[0] = o0;
          reinterpret_cast<u32x4*>(dst)[1] = o1;
        } else {
          f32x4 o0, o1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x1 = __uint_as_float(kreg[i][0][e]), x2 = __uint_as_float(kreg[i][1][e]);
            const float y1 = x1 * rc[i][e] - x2 * rs[i][e], y2 = x2 * rc[i][e] + x1 * rs[i][e];
            if (e < 2) { o0[2 * e] = y1; o0[2 * e + 1] = y2; }
            else { o1[2 * e - 4] = y1; o1[2 * e - 3] = y2; }
          }
          reinterpret_cast<f32x4*>(dst)[0] = o0;
          reinterpret_cast<f32x4*>(dst)[1] = o1;
        }
      }
      // advance the rotation to the next tile's key position
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float2 st = sm.step[kc[i] * EPC + e];
        const float c = rc[i][e], s = rs[i][e];
        rc[i][e] = c * st.x - s * st.y;
        rs[i][e] = s * st.x + c * st.y;
      }
    }
#pragma unroll
    for (int i = 0; i < C::VT; ++i) {
      if (!von[i]) continue;
      if constexpr (C::kBf16) {
        const int pr = vtask[i] / (D / 8), dc = vtask[i] % (D / 8);
        const int pos = swap_bits23(2 * pr);   // key order of the S^T register layout
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w0 = vreg[i][0][e >> 1], w1 = vreg[i][1][e >> 1];
          const uint32_t pk = (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                      : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
          const int row = dc * 8 + e;
          const int unit = (pos >> 3) ^ ((row >> 3) & 7);
          *reinterpret_cast<uint32_t*>(&sm.v[buf][row][unit * 8 + (pos & 7)]) = pk;
        }
      } else {
        const int j = vtask[i] / (D / 4), dc = vtask[i] % (D / 4);
        *reinterpret_cast<u32x4*>(&sm.v[buf][j][dc * 4]) = vreg[i][0];
      }
    }
  };

  __syncthreads();   // step table
  {
    const int rlo = stage_lo(0);
    stage_load(0, rlo);
    stage_store(0, 0, rlo);
  }
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    int rlo_next = H;
    if (t + 1 < n_kt) {
      rlo_next = stage_lo(t + 1);
      stage_load(t + 1, rlo_next);
    }

    const int64_t m_lo = (int64_t)t * kTK;
    const int64_t m_hi = min(m_lo + kTK - 1, (int64_t)p.n_kv - 1);
    int64_t dmin = 0, dmax = 0;
    if (wave_rows && tile_distance_range(n_lo, n_hi, m_lo, m_hi, causal, &dmin, &dmax)) {
      const int r_any = wave_pairs_below(w_lane, dmin);
      const int r_full = wave_pairs_below(w_lane, dmax);
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      const int64_t kbase_lane = m_lo + 4 * sh;   // key position of acc row 0 in this lane half

      // zero the cells where pair pp is outside its window
      auto drop_cells = [&](int pp) {
        int thr_lo, thr_hi;
        drop_bounds(npos, p.win.w[pp], kbase_lane, causal, kTK, &thr_lo, &thr_hi);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ko = 32 * blk + acc_row(v);
            if (ko < thr_lo || ko > thr_hi) sacc[blk][v] = 0.f;
          }
      };

      if constexpr (C::kBf16) {
        const T* krow0 = &sm.k[buf][l32][0];
        const T* krow1 = &sm.k[buf][32 + l32][0];
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          const int p0 = 8 * ks;
          if (p0 + 8 <= r_any) continue;
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow0 + 2 * (p0 + 4 * sh));
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(krow1 + 2 * (p0 + 4 * sh));
          const u32x4 qw = __builtin_bit_cast(u32x4, qop[ks]);
          const int plo = max(p0, r_any), phi_ = min(p0 + 8, r_full);
          for (int pp = plo; pp < phi_; ++pp) {
            const int u = pp - p0;
            u32x4 bw = u32x4{0, 0, 0, 0};
            if (sh == (u >> 2)) {
              const int d = u & 3;
              bw[0] = d == 0 ? qw[0] : 0u;
              bw[1] = d == 1 ? qw[1] : 0u;
              bw[2] = d == 2 ? qw[2] : 0u;
              bw[3] = d == 3 ? qw[3] : 0u;
            }
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bop, sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bop, sacc[1], 0, 0, 0);
            drop_cells(pp);
          }
          if (p0 + 8 > r_full) {
            u32x4 bw = qw;
            if (r_full > p0) {
#pragma unroll
              for (int d = 0; d < 4; ++d)
                if (p0 + 4 * sh + d < r_full) bw[d] = 0u;
            }
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bop, sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bop, sacc[1], 0, 0, 0);
          }
        }
      } else {
        const T* krow0 = &sm.k[buf][l32][0];
        const T* krow1 = &sm.k[buf][32 + l32][0];
#pragma unroll
        for (int r = 0; r < H; ++r) {
          if (r < r_any) continue;
          const float a0 = (float)krow0[2 * r + sh];
          const float a1 = (float)krow1[2 * r + sh];
          sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, qf[r], sacc[0], 0, 0, 0);
          sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, qf[r], sacc[1], 0, 0, 0);
          if (r < r_full) drop_cells(r);
        }
      }

      // causal and ragged-tail masks (cells outside the attended set)
      const bool need_mask = (causal && m_lo + kTK - 1 > n_lo) || (m_lo + kTK > p.n_kv);
      if (need_mask) {
        int thc, thr;
        hide_bounds(npos, kbase_lane, p.n_kv, causal, kTK, &thc, &thr);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ko = 32 * blk + acc_row(v);
            if (ko > thc || ko >= thr) sacc[blk][v] = -INFINITY;
          }
      }

      // online softmax (base-2, scale folded into the exponent)
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[blk][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_new - m_run) * p.scale_log2 > kRescaleLog2;
      if (__any(grow)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f((m_run - m_new) * p.scale_log2);
#pragma unroll
        for (int b = 0; b < C::ND; ++b) oacc[b] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float mb = (m_run == -INFINITY) ? 0.f : m_run * p.scale_log2;
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][v], p.scale_log2, -mb));
          sacc[blk][v] = e;
          if constexpr (!C::kBf16) lsum += e;
        }

      // O^T += V^T P^T
      if constexpr (C::kBf16) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x4 pw;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pw[i] = pack_bf16(sacc[g >> 1][8 * (g & 1) + 2 * i], sacc[g >> 1][8 * (g & 1) + 2 * i + 1]);
            // the normalizer sums the same rounded weights the PV product uses
            lsum = sum_bf16x2(pw[i], lsum);
          }
          const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
          for (int b = 0; b < C::ND; ++b) {
            const int row = 32 * b + l32;
            const int unit = (2 * g + sh) ^ ((row >> 3) & 7);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.v[buf][row][unit * 8]);
            oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop, oacc[b], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = 32 * blk + acc_row(v) + 4 * sh;
#pragma unroll
            for (int b = 0; b < C::ND; ++b) {
              const float a = (float)sm.v[buf][key][32 * b + l32];
              oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[blk][v], oacc[b], 0, 0, 0);
            }
          }
      }
      l_run += lsum;
    }

    if (t + 1 < n_kt) stage_store(t + 1, buf ^ 1, rlo_next);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const int row = w_first + l32;
  if (wave_rows && row <= w_last) {
    T* orow = obase + (int64_t)row * p.os[2];
#pragma unroll
    for (int b = 0; b < C::ND; ++b)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * b + 8 * v4 + 4 * sh;
        const float y0 = oacc[b][4 * v4] * inv, y1 = oacc[b][4 * v4 + 1] * inv;
        const float y2 = oacc[b][4 * v4 + 2] * inv, y3 = oacc[b][4 * v4 + 3] * inv;
        if constexpr (C::kBf16) {
          u32x2 w;
          w[0] = pack_bf16(y0, y1);
          w[1] = pack_bf16(y2, y3);
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        } else {
          *reinterpret_cast<f32x4*>(orow + d0) = f32x4{y0, y1, y2, y3};
        }
      }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_qblk * p.h_q * p.batch;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(kThreads);
  if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<__bf16, 128>), grid, block, 0, stream, p);
  else if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((prefill_kernel<__bf16, 64>), grid, block, 0, stream, p);
  else if (dtype == 0 && head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<float, 128>), grid, block, 0, stream, p);
  else if (dtype == 0 && head_dim == 64)
    hipLaunchKernelGGL((prefill_kernel<float, 64>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace atw
