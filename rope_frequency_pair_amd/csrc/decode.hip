// Windowed split-KV decode and its combine pass for gfx950 (MI355X).
//
// Method: "ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
// idea": for a key at distance delta from the query, the pairs whose window
// is shorter than delta contribute nothing, so that prefix of the pre-RoPE
// key row is not loaded; the rest is rotated as it is loaded.  The
// split-KV partition and the merge of per-split (max, sum, output) partials
// are the standard online-softmax merge; the window does not change them.
//
// Work layout (CDNA4 design):
//  * one workgroup = one wave = one (sequence, kv head, split); the columns
//    of S^T = K' Q'^T are the query heads that read this kv head (GQA), so the
//    key tile is read once for all of them;
//  * key tiles of 32 keys; a lane owns one 16-byte pair chunk of every 8th
//    key of the split, so its RoPE angle advances by a constant 8*theta_r per
//    tile round (rotation recurrence, re-anchored exactly every 64 rounds);
//  * the next tile's K chunks and V rows are loaded into registers while the
//    current tile is computed from LDS;
//  * partial (max, sum, unnormalised output) per split go to the caller's
//    workspace; the combine kernel merges them.
#include "device_common.h"
#include "kernels.h"

namespace atw {
namespace {

constexpr int kTK = 32;              // keys per tile
constexpr int kRounds = kTK / 8;     // K staging rounds per tile (8 keys each)
constexpr int kReanchorRounds = 64;
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
__device__ __forceinline__ constexpr int acc_row(int v) { return 8 * (v >> 2) + (v & 3); }

template <int D>
struct DSmem {
  __bf16 k[kTK][D + 8];              // rotated keys, pairs interleaved
  __bf16 v[D][kTK + 8];              // V^T, keys in S^T register order
  float2 step[D / 2];                // cos/sin of 8*theta_r
};

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
  constexpr int H = D / 2, NKS = D / 16, ND = D / 32;
  constexpr int NVT = (kTK / 2) * (D / 8) / 64;    // V staging tasks per lane
  __shared__ DSmem<D> sm;

  const int lane = threadIdx.x, sh = lane >> 5, l32 = lane & 31;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int kv_len = p.kv_len[b];
  const int64_t qpos = p.q_pos[b];
  const bool causal = p.causal != 0;
  const int chunk = (kv_len + p.splits - 1) / p.splits;
  const int k_begin = min(split * chunk, kv_len), k_end = min(k_begin + chunk, kv_len);

  const int g0 = p.kv_first[kvh], G = p.kv_first[kvh + 1] - g0;
  const int w_lane = lane < H ? p.win.w[lane] : kWindowInf;

  const __bf16* kbase = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* vbase = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];

  if (lane < H) {
    float s, c;
    rope_sincos(8, p.win.phi[lane], &s, &c);
    sm.step[lane] = make_float2(c, s);
  }

  // query operand: column l32 = the l32-th query head of this kv head
  bf16x8 qop[NKS];
  {
    const bool valid = l32 < G;
    const int qh = valid ? p.qh_of_kv[g0 + l32] : 0;
    const __bf16* qrow = (const __bf16*)p.q + b * p.qs[0] + qh * p.qs[1];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int r0 = 8 * ks + 4 * sh;
      u32x4 packed = u32x4{0, 0, 0, 0};
      if (valid) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(qrow + r0);
        const u32x2 c2 = *reinterpret_cast<const u32x2*>(qrow + H + r0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x1 = (u & 1) ? bf16_hi(a[u >> 1]) : bf16_lo(a[u >> 1]);
          const float x2 = (u & 1) ? bf16_hi(c2[u >> 1]) : bf16_lo(c2[u >> 1]);
          float s, c;
          rope_sincos(qpos, p.win.phi[r0 + u], &s, &c);
          packed[u] = pack_bf16(x1 * c - x2 * s, x2 * c + x1 * s);
        }
      }
      qop[ks] = __builtin_bit_cast(bf16x8, packed);
    }
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K staging: lane = (key offset kj in 0..7, pair chunk kc in 0..7 of H/8)
  constexpr int NCH = H / 8;
  const int kj = lane / NCH;                  // D=128: 0..7; D=64: 0..15
  const int kc = lane % NCH;
  constexpr int KEYS_PER_ROUND = 64 / NCH;    // 8 (D=128) or 16 (D=64)
  constexpr int ROUNDS = kTK / KEYS_PER_ROUND;
  float rc[8], rs[8];
  u32x4 kreg[ROUNDS][2];
  u32x4 vreg[NVT][2];

  const int n_tiles = (k_end - k_begin + kTK - 1) / kTK;

  auto tile_lo = [&](int t) -> int {     // first pair needed by any key of tile t
    const int64_t m_lo = k_begin + (int64_t)t * kTK;
    const int64_t m_hi = min(m_lo + kTK - 1, (int64_t)k_end - 1);
    int64_t dmin = 0, dmax = 0;
    if (!tile_distance_range(qpos, qpos, m_lo, m_hi, causal, &dmin, &dmax)) return H;
    return wave_pairs_below(w_lane, dmin) & ~7;
  };

  auto load_tile = [&](int t, int rlo) {
    const int64_t m0 = k_begin + (int64_t)t * kTK;
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int64_t m = m0 + KEYS_PER_ROUND * i + kj;
      if ((kc + 1) * 8 > rlo && m < k_end) {
        const __bf16* src = kbase + m * p.ks[2] + kc * 8;
        kreg[i][0] = *reinterpret_cast<const u32x4*>(src);
        kreg[i][1] = *reinterpret_cast<const u32x4*>(src + H);
      } else {
        kreg[i][0] = u32x4{0, 0, 0, 0};
        kreg[i][1] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int task = lane + 64 * i;
      const int pr = task / (D / 8), dc = task % (D / 8);
      const int64_t m = m0 + 2 * pr;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (m + e < k_end)
          vreg[i][e] = *reinterpret_cast<const u32x4*>(vbase + (m + e) * p.vs[2] + dc * 8);
        else
          vreg[i][e] = u32x4{0, 0, 0, 0};
      }
    }
  };

  int round_ix = 0;   // K staging rounds done so far (drives the recurrence)
  auto store_tile = [&](int t, int rlo) {
    const int64_t m0 = k_begin + (int64_t)t * kTK;
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int64_t m = m0 + KEYS_PER_ROUND * i + kj;
      if (round_ix % kReanchorRounds == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_sincos(m, p.win.phi[kc * 8 + e], &rs[e], &rc[e]);
      }
      if ((kc + 1) * 8 > rlo) {
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wa = kreg[i][0][e >> 1], wb = kreg[i][1][e >> 1];
          const float x1 = (e & 1) ? bf16_hi(wa) : bf16_lo(wa);
          const float x2 = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
          const uint32_t pk = pack_bf16(x1 * rc[e] - x2 * rs[e], x2 * rc[e] + x1 * rs[e]);
          if (e < 4) o0[e] = pk; else o1[e - 4] = pk;
        }
        __bf16* dst = &sm.k[KEYS_PER_ROUND * i + kj][16 * kc];
        reinterpret_cast<u32x4*>(dst)[0] = o0;
        reinterpret_cast<u32x4*>(dst)[1] = o1;
      }
      // advance by KEYS_PER_ROUND keys: step table holds 8*theta; D=64 needs 16*theta
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float2 st = sm.step[kc * 8 + e];
        if (KEYS_PER_ROUND == 16) st = make_float2(st.x * st.x - st.y * st.y, 2.f * st.x * st.y);
        const float c = rc[e], s = rs[e];
        rc[e] = c * st.x - s * st.y;
        rs[e] = s * st.x + c * st.y;
      }
      ++round_ix;
    }
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int task = lane + 64 * i;
      const int pr = task / (D / 8), dc = task % (D / 8);
      const int pos = swap_bits23(2 * pr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vreg[i][0][e >> 1], w1 = vreg[i][1][e >> 1];
        const uint32_t pk = (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                    : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        const int row = dc * 8 + e;
        const int unit = (pos >> 3) ^ ((row >> 2) & 3);
        *reinterpret_cast<uint32_t*>(&sm.v[row][unit * 8 + (pos & 7)]) = pk;
      }
    }
  };

  __syncthreads();   // step table
  int rlo = n_tiles > 0 ? tile_lo(0) : H;
  if (n_tiles > 0) load_tile(0, rlo);

  for (int t = 0; t < n_tiles; ++t) {
    store_tile(t, rlo);
    __syncthreads();
    const int rlo_next = (t + 1 < n_tiles) ? tile_lo(t + 1) : H;
    if (t + 1 < n_tiles) load_tile(t + 1, rlo_next);

    const int64_t m_lo = k_begin + (int64_t)t * kTK;
    const int64_t m_hi = min(m_lo + kTK - 1, (int64_t)k_end - 1);
    int64_t dmin = 0, dmax = 0;
    if (tile_distance_range(qpos, qpos, m_lo, m_hi, causal, &dmin, &dmax)) {
      const int r_any = wave_pairs_below(w_lane, dmin);
      const int r_full = wave_pairs_below(w_lane, dmax);
      f32x16 sacc = f32x16{};
      const int64_t kbl = m_lo + 4 * sh;
      const __bf16* krow = &sm.k[l32][0];

      auto drop_cells = [&](int pp) {
        int thr_lo, thr_hi;
        drop_bounds((int)qpos, p.win.w[pp], (int)kbl, causal, kTK, &thr_lo, &thr_hi);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ko = acc_row(v);
          if (ko < thr_lo || ko > thr_hi) sacc[v] = 0.f;
        }
      };

#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int p0 = 8 * ks;
        if (p0 + 8 <= r_any) continue;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 2 * (p0 + 4 * sh));
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
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bw), sacc, 0, 0, 0);
          drop_cells(pp);
        }
        if (p0 + 8 > r_full) {
          u32x4 bw = qw;
          if (r_full > p0) {
#pragma unroll
            for (int d = 0; d < 4; ++d)
              if (p0 + 4 * sh + d < r_full) bw[d] = 0u;
          }
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bw), sacc, 0, 0, 0);
        }
      }

      // keys past the end of the split / not visible
      if (m_lo + kTK > k_end || (causal && m_lo + kTK - 1 > qpos)) {
        int thc, thr;
        hide_bounds((int)qpos, (int)kbl, k_end, causal, kTK, &thc, &thr);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ko = acc_row(v);
          if (ko > thc || ko >= thr) sacc[v] = -INFINITY;
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_new - m_run) * p.scale_log2 > kRescaleLog2;
      if (__any(grow)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f((m_run - m_new) * p.scale_log2);
#pragma unroll
        for (int i = 0; i < ND; ++i) oacc[i] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float mb = (m_run == -INFINITY) ? 0.f : m_run * p.scale_log2;
      float lsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sacc[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.scale_log2, -mb));

#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4 pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = pack_bf16(sacc[8 * g + 2 * i], sacc[8 * g + 2 * i + 1]);
          lsum = sum_bf16x2(pw[i], lsum);     // normalizer of the rounded weights
        }
        const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int bd = 0; bd < ND; ++bd) {
          const int row = 32 * bd + l32;
          const int unit = (2 * g + sh) ^ ((row >> 2) & 3);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.v[row][unit * 8]);
          oacc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop, oacc[bd], 0, 0, 0);
        }
      }
      l_run += lsum;
    }
    rlo = rlo_next;
    __syncthreads();   // LDS reads done before the next store
  }

  // partial result of this split: [m (raw score units), l, -, -, o[D]] per query head
  const float l_tot = half_swap_sum(l_run);
  if (l32 < G) {
    const int qh = p.qh_of_kv[g0 + l32];
    float* w = p.ws + (((int64_t)b * p.h_q + qh) * p.splits + split) * (D + 4);
    if (sh == 0) {
      w[0] = m_run;
      w[1] = l_tot;
    }
#pragma unroll
    for (int bd = 0; bd < ND; ++bd)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * bd + 8 * v4 + 4 * sh;
        *reinterpret_cast<f32x4*>(w + 4 + d0) =
            f32x4{oacc[bd][4 * v4], oacc[bd][4 * v4 + 1], oacc[bd][4 * v4 + 2], oacc[bd][4 * v4 + 3]};
      }
  }
}

// Merge the splits of one (sequence, query head): standard online-softmax
// merge of (max, sum, unnormalised output) partials.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const DecodeParams p) {
  const int qh = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* w = p.ws + ((int64_t)b * p.h_q + qh) * p.splits * (D + 4);
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, w[s * (D + 4)]);
  float l = 0.f, acc = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float ms = w[s * (D + 4)];
    if (ms == -INFINITY) continue;
    const float a = exp2f((ms - m) * p.scale_log2);
    l += a * w[s * (D + 4) + 1];
    acc += a * w[s * (D + 4) + 4 + d];
  }
  __bf16* o = (__bf16*)p.o + b * p.os[0] + qh * p.os[1];
  o[d] = (__bf16)(acc / l);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream) {
  dim3 grid((unsigned)p.splits, (unsigned)p.h_kv, (unsigned)p.batch);
  dim3 cgrid((unsigned)p.h_q, (unsigned)p.batch);
  if (head_dim == 128) {
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL((decode_combine_kernel<128>), cgrid, dim3(128), 0, stream, p);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL((decode_combine_kernel<64>), cgrid, dim3(64), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace atw
