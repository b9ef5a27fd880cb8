// Tile plans and per-tile pruned-term counts computed on the GPU with the
// same device code the attention kernels use for their per-tile pair ranges
// (span32 -- the prefill kernels' distance range, taken whenever positions
// are below 2^30 as in every prefill call -- else the 64-bit
// tile_distance_range the decode kernels use; wave_pairs_below) and per-cell
// masks (drop_bounds, hide_bounds).  "ATFlash — Per-RoPE-Wavelength Attention Windows", README,
// "Porting to something else": the retained prefix per key tile; "The idea":
// the pruned share is input independent.
#include "device_common.h"
#include "kernels.h"

namespace atw {
namespace {

__global__ __launch_bounds__(64) void plan_kernel(const PlanParams p) {
  const int lane = threadIdx.x;
  const int w_lane = lane < p.h ? p.win.w[lane] : kWindowInf;
  const int64_t n_tiles = p.n_qt * p.n_kt;
  const int64_t n_end = p.n_kv;
  const bool small = p.q_pos0 + p.n_q <= (int64_t(1) << 30) && p.n_kv <= (int64_t(1) << 30);
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t a = tile / p.n_kt, b = tile % p.n_kt;
    const int64_t r_lo_row = a * p.tile_q;
    const int64_t rows = min((int64_t)p.tile_q, p.n_q - r_lo_row);
    const int64_t n_lo = p.q_pos0 + r_lo_row, n_hi = n_lo + rows - 1;
    const int64_t m_lo = b * p.tile_k;
    const int64_t cols = min((int64_t)p.tile_k, p.n_kv - m_lo);
    const int64_t m_hi = m_lo + cols - 1;
    int64_t dmin = 0, dmax = 0;
    bool any;
    if (small) {
      int d0 = 0, d1 = 0;
      any = span32((int)n_lo, (int)n_hi, (int)m_lo, (int)m_hi, p.causal != 0, &d0, &d1);
      dmin = d0;
      dmax = d1;
    } else {
      any = tile_distance_range(n_lo, n_hi, m_lo, m_hi, p.causal != 0, &dmin, &dmax);
    }
    int r_any = -1, r_full = -1;
    if (any) {
      r_any = wave_pairs_below(w_lane, dmin);
      r_full = wave_pairs_below(w_lane, dmax);
    }
    int64_t cnt = 0;
    if (any) {
      for (int64_t cell = lane; cell < rows * cols; cell += 64) {
        const int64_t n = n_lo + cell / cols;
        const int ko = (int)(cell % cols);
        int fut, end;
        hide_bounds((int)n, (int)m_lo, (int)n_end, p.causal != 0, p.tile_k, &fut, &end);
        if (ko > fut || ko >= end) continue;            // not a visible cell
        int c = r_any;                                   // pairs below r_any: never computed
        for (int pp = r_any; pp < r_full; ++pp) {
          int lo, hi;
          drop_bounds((int)n, p.win.w[pp], (int)m_lo, p.causal != 0, p.tile_k, &lo, &hi);
          if (ko < lo || ko > hi) ++c;
        }
        cnt += c;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) {
      p.plan[tile * 2] = r_any;
      p.plan[tile * 2 + 1] = r_full;
      p.pruned[tile] = cnt;
    }
  }
}

}  // namespace

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  const int64_t n_tiles = p.n_qt * p.n_kt;
  if (n_tiles <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)min(n_tiles, (int64_t)65536);
  hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace atw
