// Windowed causal prefill for fp32 inputs, gfx950 (MI355X).
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
//  * workgroups are dispatched largest causal blocks first, and the ones
//    resident on one XCD (workgroup i runs on XCD i mod 8) are consecutive
//    blocks of one (batch, kv head), so they share key/value tiles in its L2
//    (whole kv heads per XCD when they divide evenly, else balanced rounds);
//  * scores are computed transposed, S^T = K' Q'^T, with
//    v_mfma_f32_32x32x2f32 (one pair-dimension per MFMA), so each lane holds
//    16 keys of one query column and the row max / sum are mostly in-lane;
//    lanes l and l+32 share a query (lane half s takes dim r or r + h of
//    pair r);
//  * the pairs are taken in ascending order from the tile's first needed
//    pair; pairs that are in the window for some cells of a wave's tile and
//    not for others ("partial" pairs) come first, and after each such pair
//    the cells beyond its window are reset to zero; because windows grow
//    with r, this leaves exactly the kept partial terms;
//  * O^T += V^T P^T one key per MFMA, P^T straight from the S^T registers;
//  * waves 0-3 run each tile as [QK^T, softmax, PV, RoPE staging of the
//    next tile] and waves 4-7 as [staging, QK^T, softmax, PV], so on each
//    SIMD the MFMA stretches of one wave meet the VALU stretches of the
//    other; one workgroup barrier per tile;
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

template <int D>
struct Cfg {
  static constexpr int H = D / 2;
  // K staging: thread = (key tid/8, pair group tid%8) of PPT pairs
  static constexpr int PPT = H / 8;
  static constexpr int KROW = D + 4;      // K' row (pairs interleaved), 16-byte pad
  static constexpr int VROW = D + 4;      // V row, row-major as in memory
  static constexpr int NVT = D * 4 / 128; // 16-byte V chunks per thread per tile
  static constexpr int ND = D / 32;       // 32-wide head-dim blocks
};

template <int D>
struct Smem {
  float k[2][kTK][Cfg<D>::KROW];
  float v[2][kTK][Cfg<D>::VROW];
};

// Key offset (within a 32-key block, before + 4*s) of accumulator register v
// in the 32x32 MFMA output layout.
__device__ __forceinline__ constexpr int acc_row(int v) { return 8 * (v >> 2) + (v & 3); }

// Register chunks of 8, 16 or 32 bytes.
template <int BYTES>
struct Chunk {
  static constexpr int N = BYTES / 4;
  uint32_t w[N];
};
template <int BYTES>
__device__ __forceinline__ Chunk<BYTES> load_chunk(const void* p) {
  Chunk<BYTES> c;
  if constexpr (BYTES == 8) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    c.w[0] = x[0];
    c.w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const u32x4 x = reinterpret_cast<const u32x4*>(p)[i];
      c.w[4 * i] = x[0];
      c.w[4 * i + 1] = x[1];
      c.w[4 * i + 2] = x[2];
      c.w[4 * i + 3] = x[3];
    }
  }
  return c;
}
template <int BYTES>
__device__ __forceinline__ Chunk<BYTES> zero_chunk() {
  Chunk<BYTES> c;
#pragma unroll
  for (int i = 0; i < BYTES / 4; ++i) c.w[i] = 0u;
  return c;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillParams p) {
  using C = Cfg<D>;
  using T = float;
  constexpr int H = C::H;
  constexpr int PPT = C::PPT;
  constexpr int KBYTES = PPT * 4;                              // bytes per half row per K task
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sh = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;   // 0: waves 0-3, 1: waves 4-7 (one phase later)

  // ---- work item.  The list (batch, kv head, query block descending, query
  // head) is mapped onto the XCDs (XCD x runs workgroups x, x+8, ...):
  //  * when the (batch, kv head) groups split evenly over the 8 XCDs, XCD x
  //    takes a contiguous eighth of the list (whole groups: its L2 serves
  //    only its own kv heads);
  //  * otherwise the list is dealt in rounds of 8 x 32 entries, XCD x taking
  //    32 consecutive entries per round, which balances the causal work;
  // the last partial round keeps the identity order.
  int bb, hq, qb, kvh;
  {
    constexpr int kRound = 32;
    const int W = p.n_qblk * p.h_q * p.batch;
    const int idx = (int)blockIdx.x, x = idx & 7, li = idx >> 3;
    int pos;
    if ((p.batch * p.n_kv_heads) % 8 == 0 && W % 8 == 0) {
      pos = x * (W >> 3) + li;
    } else {
      const int full = W / (8 * kRound);
      const int round = li / kRound;
      pos = (round < full) ? round * 8 * kRound + x * kRound + li % kRound : idx;
    }
    const int per_b = p.n_qblk * p.h_q;
    bb = pos / per_b;
    const int r = pos - bb * per_b;
    int j = 0;
    while ((int)p.kv_first[j + 1] * p.n_qblk <= r) ++j;
    const int r2 = r - (int)p.kv_first[j] * p.n_qblk;
    const int G = p.kv_first[j + 1] - p.kv_first[j];
    qb = p.n_qblk - 1 - r2 / G;
    hq = p.qh_of_kv[p.kv_first[j] + r2 % G];
    kvh = j;
  }

  const T* qbase = (const T*)p.q + bb * p.qs[0] + hq * p.qs[1];
  const T* kbase = (const T*)p.k + bb * p.ks[0] + kvh * p.ks[1];
  const T* vbase = (const T*)p.v + bb * p.vs[0] + kvh * p.vs[1];
  T* obase = (T*)p.o + bb * p.os[0] + hq * p.os[1];

  const bool causal = p.causal != 0;
  const int n_kv = p.n_kv;
  const int i0 = qb * kPrefillBlockRows;
  const int g_last = min(i0 + kPrefillBlockRows - 1, p.n_q - 1);
  const int w_first = i0 + wave * kRowsW;
  const int w_last = min(w_first + kRowsW - 1, p.n_q - 1);
  const bool wave_rows = w_first <= w_last;
  const int n_lo = p.q_pos0 + w_first, n_hi = p.q_pos0 + w_last;
  const int gn_lo = p.q_pos0 + i0, gn_hi = p.q_pos0 + g_last;
  const int qrow = min(w_first + l32, p.n_q - 1);
  const int npos = p.q_pos0 + qrow;
  const int w_lane = lane < H ? p.win.w[lane] : kWindowInf;

  // ---- query: load, rotate at its position, keep as MFMA operand
  const T* qrow_ptr = qbase + (int64_t)qrow * p.qs[2];
  float qf[H];   // lane half s: dim r (s = 0) or r + h (s = 1) of pair r, rotated
#pragma unroll
  for (int r = 0; r < H; ++r) {
    const float x1 = qrow_ptr[r], x2 = qrow_ptr[H + r];
    float s, c;
    rope_sincos(npos, p.win.phi[r], &s, &c);
    qf[r] = sh ? (x2 * c + x1 * s) : (x1 * c - x2 * s);
  }

  f32x16 oacc[C::ND];
#pragma unroll
  for (int b = 0; b < C::ND; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = causal ? min(n_kv, gn_hi + 1) : n_kv;
  const int n_kt = (kv_end + kTK - 1) / kTK;

  // ---- staging tasks (fixed over tiles)
  // K: wave w stages pair chunk kc (PPT pairs) of all 64 keys of a tile, lane =
  // key, so a chunk that the window prunes is skipped by a whole wave; chunks
  // are interleaved between the two wave groups to keep them balanced.
  const int kj = lane, kc = ((wave & 3) << 1) | (wave >> 2);
  const T* ksrc = kbase + (int64_t)kj * p.ks[2] + kc * PPT;
  const int64_t kstep = (int64_t)kTK * p.ks[2];
  const int koff0 = kj * C::KROW + 2 * kc * PPT;   // LDS element offset of the K' writes (pairs interleaved)
  // RoPE step over one key tile (64*theta_r) for the wave's pairs: uniform
  float st_c[PPT], st_s[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    float s, c;
    rope_sincos(kTK, p.win.phi[kc * PPT + e], &s, &c);
    st_c[e] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));
    st_s[e] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s)));
  }
  // V: row-major 16-byte chunks, task = tid + 512*i -> (key, chunk)
  constexpr int VCH = D * 4 / 16;                // 16-byte chunks per V row
  const T* vsrc[C::NVT];
  int voff[C::NVT], vkey[C::NVT];
#pragma unroll
  for (int i = 0; i < C::NVT; ++i) {
    const int task = tid + kThreads * i;
    vkey[i] = task / VCH;
    const int ch = task % VCH;
    vsrc[i] = vbase + (int64_t)vkey[i] * p.vs[2] + ch * 4;
    voff[i] = vkey[i] * C::VROW + ch * 4;
  }
  const int64_t vstep = (int64_t)kTK * p.vs[2];

  float rc[PPT], rs[PPT];          // cos/sin of the RoPE angle of the next staged K tile
  Chunk<KBYTES> kreg0, kreg1;
  Chunk<16> vreg[C::NVT];

  // WG-wide first pair needed in key tile t (the staging start)
  auto stage_lo = [&](int t) -> int {
    const int m_lo = t * kTK;
    const int m_hi = min(m_lo + kTK - 1, n_kv - 1);
    int64_t dmin = 0, dmax = 0;
    if (!tile_distance_range(gn_lo, gn_hi, m_lo, m_hi, causal, &dmin, &dmax)) return H;
    return wave_pairs_below(w_lane, dmin);
  };

  auto load_k = [&](int t) {
    const int m = t * kTK + kj;
    if ((kc + 1) * PPT > stage_lo(t)) {          // uniform over the wave
      if (m < n_kv) {
        const T* src = ksrc + t * kstep;
        kreg0 = load_chunk<KBYTES>(src);
        kreg1 = load_chunk<KBYTES>(src + H);
      } else {
        kreg0 = zero_chunk<KBYTES>();
        kreg1 = zero_chunk<KBYTES>();
      }
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::NVT; ++i)
      vreg[i] = (t * kTK + vkey[i] < n_kv) ? load_chunk<16>(vsrc[i] + t * vstep) : zero_chunk<16>();
  };
  auto write_k = [&](int t) {
    const int m = t * kTK + kj;
    if (t % kReanchor == 0) {
#pragma unroll
      for (int e = 0; e < PPT; ++e) rope_sincos(m, p.win.phi[kc * PPT + e], &rs[e], &rc[e]);
    }
    if ((kc + 1) * PPT > stage_lo(t)) {          // uniform over the wave
      T* dst = &sm.k[t & 1][0][0];
      float y[2 * PPT];
#pragma unroll
      for (int e = 0; e < PPT; ++e) {
        const float x1 = __uint_as_float(kreg0.w[e]), x2 = __uint_as_float(kreg1.w[e]);
        y[2 * e] = x1 * rc[e] - x2 * rs[e];
        y[2 * e + 1] = x2 * rc[e] + x1 * rs[e];
      }
#pragma unroll
      for (int i = 0; i < PPT / 2; ++i)
        reinterpret_cast<f32x4*>(dst + koff0)[i] = f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
    }
    // advance the rotation to the next tile's key position
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const float c = rc[e], s = rs[e];
      rc[e] = c * st_c[e] - s * st_s[e];
      rs[e] = s * st_c[e] + c * st_s[e];
    }
  };
  auto write_v = [&](int t) {
    T* dst = &sm.v[t & 1][0][0];
#pragma unroll
    for (int i = 0; i < C::NVT; ++i)
      *reinterpret_cast<u32x4*>(dst + voff[i]) = u32x4{vreg[i].w[0], vreg[i].w[1], vreg[i].w[2], vreg[i].w[3]};
  };

  // ---- prologue: tile 0 by everyone; waves 4-7 also load tile 1
  load_k(0);
  load_v(0);
  write_k(0);
  write_v(0);
  if (grp == 1 && n_kt > 1) {
    load_k(1);
    load_v(1);
  }
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    if (grp == 0) {
      if (t + 1 < n_kt) {
        load_k(t + 1);
        load_v(t + 1);
      }
    } else {
      if (t + 1 < n_kt) {
        write_k(t + 1);
        write_v(t + 1);
      }
      if (t + 2 < n_kt) {
        load_k(t + 2);
        load_v(t + 2);
      }
    }

    const int m_lo = t * kTK;
    const int m_hi = min(m_lo + kTK - 1, n_kv - 1);
    int64_t dmin = 0, dmax = 0;
    if (wave_rows && tile_distance_range(n_lo, n_hi, m_lo, m_hi, causal, &dmin, &dmax)) {
      const int r_any = wave_pairs_below(w_lane, dmin);
      const int r_full = wave_pairs_below(w_lane, dmax);
      const int kbase_lane = m_lo + 4 * sh;
      f32x16 sacc[2];
      const T* kt = &sm.k[t & 1][0][0];

      // reset the cells of x beyond the window of partially windowed pair pp
      auto drop_cells = [&](f32x16 (&x)[2], int pp) {
        int thr_lo, thr_hi;
        drop_bounds(npos, p.win.w[pp], kbase_lane, causal, kTK, &thr_lo, &thr_hi);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ko = 32 * blk + acc_row(v);
            if (ko < thr_lo || ko > thr_hi) x[blk][v] = 0.f;
          }
      };

      const T* krow0 = kt + l32 * C::KROW + sh;
      const T* krow1 = krow0 + 32 * C::KROW;
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
#pragma unroll
      for (int r = 0; r < H; ++r) {
        if (r < r_any) continue;
        const float a0 = krow0[2 * r];
        const float a1 = krow1[2 * r];
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, qf[r], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, qf[r], sacc[1], 0, 0, 0);
        if (r < r_full) drop_cells(sacc, r);
      }

      // causal and ragged-tail masks (cells outside the attended set)
      const bool need_mask = (causal && m_lo + kTK - 1 > n_lo) || (m_lo + kTK > n_kv);
      if (need_mask) {
        int thc, thr;
        hide_bounds(npos, kbase_lane, n_kv, causal, kTK, &thc, &thr);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ko = 32 * blk + acc_row(v);
            if (ko > thc || ko >= thr) sacc[blk][v] = -INFINITY;
          }
      }

      // online softmax (base 2, scale folded into the exponent)
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[blk][v]);
      mx = half_swap_max(mx);
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
      const T* vt = &sm.v[t & 1][0][0];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][v], p.scale_log2, -mb));
          lsum += e;
          const int key = 32 * blk + acc_row(v) + 4 * sh;
#pragma unroll
          for (int b = 0; b < C::ND; ++b) {
            const float a = vt[key * C::VROW + 32 * b + l32];
            oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, e, oacc[b], 0, 0, 0);
          }
        }
      l_run += lsum;
    }

    if (grp == 0 && t + 1 < n_kt) {
      write_k(t + 1);
      write_v(t + 1);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l
  const float l_tot = half_swap_sum(l_run);
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
        *reinterpret_cast<f32x4*>(orow + d0) = f32x4{y0, y1, y2, y3};
      }
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_qblk * p.h_q * p.batch;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(kThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<128>), grid, block, 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL((prefill_kernel<64>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace atw
