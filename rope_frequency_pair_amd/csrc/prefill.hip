// Windowed causal prefill, bf16, for gfx950 (MI355X).
//
// Method: "ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
// idea" and "Porting to something else": the window is a slice of the
// query-key contraction axis.  For a key tile, the pairs whose window is
// shorter than the tile's smallest query-key distance are never needed, so
// that part of the key tile is never loaded and its products are never
// issued.  The online softmax (running max, normalizer) is the ordinary one.
//
// Two kernels (designed for CDNA4, not taken from the pages):
//
//  range_kernel -- once per call, the largest |k| and |v| of each chunk of
//    keys of every (batch, kv head), from which the packing and attention
//    kernels derive the same power-of-two operand scales.
//
//  pack_kv_kernel -- once per call, rotates every key at its position
//    (RoPE) and writes K' and V in the order the matrix-core operands are
//    read: a 64-key tile is a run of 1 KB blocks, one block per (operand,
//    wave-wide read), lane l's 16 bytes at l * 16.  The pages fuse RoPE into
//    the attention loads; here every key tile is read by every query block
//    of its head, so rotating it there repeats the same work hundreds of
//    times on the vector ALUs, which bound the loop on this GPU.  One pass
//    over K and V (a fraction of a percent of the attention time) removes it.
//
//  prefill_bf16_kernel -- one workgroup = consecutive query rows of one
//    query head, 32 per wave (head_dim 128: 12 waves, 384 rows; head_dim 64:
//    8 waves, 256 rows); key tiles of 64 keys, double-buffered in LDS:
//  * staging copies 1 KB blocks straight from global memory into LDS
//    (global_load_lds_dwordx4, no registers on the way; wave w copies blocks
//    w, w + waves, ...), one tile ahead; K' blocks of k-steps that the window
//    prunes for the whole workgroup are not copied;
//  * workgroups are dispatched largest causal blocks first, and the ones
//    resident on one XCD (workgroup i runs on XCD i mod 8) are consecutive
//    blocks of one (batch, kv head), so they share K'/V tiles in its L2;
//  * scores are computed transposed, S^T = K' Q'^T, with
//    v_mfma_f32_32x32x16_f16, so each lane holds 16 keys of one query
//    column and the row max / sum are mostly in-lane; lanes l and l+32 share
//    a query;
//  * the contraction axis is ordered pair by pair ((r, r+h) adjacent): one
//    k-step of 16 covers 8 whole pairs, so the retained pairs [r, h) are a
//    contiguous range of k-steps;
//  * per tile and wave: pairs that are in the window for some cells of the
//    tile and not for others ("partial" pairs) go one pair per MFMA, and
//    after each such pair the cells beyond its window are reset to zero;
//    because windows grow with r, this leaves exactly the kept partial terms
//    (head_dim 64: first, in the score accumulator itself; head_dim 128: in a
//    separate accumulator added afterwards); the k-step holding the first
//    fully kept pair (its partial slots masked out of the query operand) and
//    the fully kept k-steps above it complete the scores;
//  * O^T += V^T P^T with P^T taken straight from the S^T registers (V is
//    packed in the key order that register layout produces);
//  * operands are fp16 (v_mfma_f32_32x32x16_f16, the bf16 rate on gfx950,
//    3 more mantissa bits than bf16): rotated queries and keys, V and the
//    softmax weights P.  A range pass finds, per (batch, kv head), the largest
//    |k| and |v|; where they reach 2^14 the packed K' / V are scaled by a
//    power of two that is undone exactly in fp32 (key scale folded into the
//    query operand, value scale into the epilogue), so any bf16 input fits;
//    the query operand carries its own per-wave power of two the same way;
//  * scores are kept relative to a per-row reference r, in base-2 units: the
//    query operand holds softmax_scale * log2(e), and the first QK^T MFMA of
//    a tile starts from -r instead of zero, so P = exp2(S) needs no per-score
//    arithmetic.  r trails the running max by 6 (P <= 2^14 stays in fp16 and
//    small weights stay out of its subnormals) and is raised only when a score
//    passes it by more than 14 (lazy rescale);
//  * one workgroup barrier per tile; tile geometry (distances, pair ranges)
//    is wave-uniform and runs on the scalar unit; causal / non-causal and
//    dense / block-sparse are separate instantiations, so neither is tested
//    in the loop;
//  * head_dim 128 runs three waves per SIMD (one workgroup of 12 waves per
//    CU: 160 KB of LDS, at most 168 registers), which hides more of each
//    wave's dependency stalls than two; to fit the registers, its query
//    operands are read from the per-wave LDS copy at every k-step.  head_dim
//    64 asks for four waves per SIMD (two workgroups of 8 waves per CU: 64 KB
//    of LDS and at most 128 registers each), query operands in registers.
#include "device_common.h"
#include "kernels.h"

namespace atw {
namespace {

constexpr int kRowsW = 32;
constexpr int kTK = kPrefillTileK;
constexpr float kRefLag = 6.0f;       // reference r = running max - 6 (base 2)
constexpr float kRaise = 14.0f;       // raise r when a score passes it by more

// Power-of-two scales of one (batch, kv head): the range pass's chunk maxima
// (bf16 magnitude bits of K and V) reduced by one wave.  Wave-uniform.
__device__ __forceinline__ void head_range_exps(const uint32_t* range, int64_t head, int* ek, int* ev) {
  const int lane = threadIdx.x & 63;
  uint32_t mk = 0, mv = 0;
  if (lane < kRangeChunks) {
    const u32x2 m = *reinterpret_cast<const u32x2*>(range + (head * kRangeChunks + lane) * 2);
    mk = m[0];
    mv = m[1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
    mv = max(mv, (uint32_t)__shfl_xor((int)mv, o));
  }
  *ek = __builtin_amdgcn_readfirstlane(range_exp_of_bf16(mk));
  *ev = __builtin_amdgcn_readfirstlane(range_exp_of_bf16(mv));
}

template <int D>
struct PCfg {
  static constexpr int H = D / 2;
  static constexpr int NKS = D / 16;      // QK^T k-steps (8 pairs each)
  static constexpr int ND = D / 32;       // 32-wide head-dim blocks of O^T
  static constexpr int KBLK = 2 * NKS;    // K' blocks per tile: (k-step, 32-key block)
  static constexpr int VBLK = 4 * ND;     // V blocks per tile: (head-dim block, 16-key group)
  // waves per workgroup: head_dim 128 runs three waves per SIMD (12 waves,
  // 384 rows, 160 KB of LDS), head_dim 64 four (two workgroups of 8 waves)
  static constexpr int WAVES = prefill_bf16_waves(D);
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BLOCK_ROWS = kRowsW * WAVES;
  static constexpr int KPW = (KBLK + WAVES - 1) / WAVES;   // staging blocks per wave
  static constexpr int VPW = (VBLK + WAVES - 1) / WAVES;
  // head_dim 128: query operands read from the per-wave LDS copy at every
  // k-step (keeping them in registers would leave too few for three waves)
  static constexpr bool Q_IN_LDS = D == 128;
};

// Element offset of the 8 bf16 values lane `lane` reads from operand block
// `blk` of a packed tile.
__device__ __forceinline__ int blk_off(int blk, int lane) { return (blk * 64 + lane) * 8; }

// Key offset (within a 32-key block, before + 4*s) of accumulator register v
// in the 32x32 MFMA output layout.
__device__ __forceinline__ constexpr int acc_row(int v) { return 8 * (v >> 2) + (v & 3); }

// Key (within a 64-key tile) of slot j of lane half s in PV key group g: the
// order in which the S^T accumulator registers hold the keys.
__device__ __forceinline__ constexpr int pv_key(int g, int s, int j) {
  return 32 * (g >> 1) + 16 * (g & 1) + 8 * (j >> 2) + 4 * s + (j & 3);
}

// Largest |k| and |v| (bf16 magnitude bits) over keys [c * per, (c+1) * per)
// of one (batch, kv head), per = ceil(n_kv / kRangeChunks).
template <int D>
__global__ __launch_bounds__(256) void range_kernel(const PackParams p) {
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  __shared__ uint32_t red[2][4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int per = (p.n_kv + kRangeChunks - 1) / kRangeChunks;
  const int m0 = min(c * per, p.n_kv), m1 = min(m0 + per, p.n_kv);
  const __bf16* kb = (const __bf16*)p.k + b * p.ks[0] + h * p.ks[1];
  const __bf16* vb = (const __bf16*)p.v + b * p.vs[0] + h * p.vs[1];
  uint32_t mk = 0, mv = 0;
  for (int i = tid; i < (m1 - m0) * CPR; i += 256) {
    const int m = m0 + i / CPR, ch = i % CPR;
    mk = max_mag_bf16x8(*reinterpret_cast<const u32x4*>(kb + (int64_t)m * p.ks[2] + ch * 8), mk);
    mv = max_mag_bf16x8(*reinterpret_cast<const u32x4*>(vb + (int64_t)m * p.vs[2] + ch * 8), mv);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, o));
    mv = max(mv, (uint32_t)__shfl_xor((int)mv, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mk;
    red[1][tid >> 6] = mv;
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t head = (int64_t)b * p.h_kv + h;
    u32x2 out;
    out[0] = max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3]));
    out[1] = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    *reinterpret_cast<u32x2*>(p.range + (head * kRangeChunks + c) * 2) = out;
  }
}

template <int D>
__global__ __launch_bounds__(256) void pack_kv_kernel(const PackParams p) {
  using C = PCfg<D>;
  constexpr int H = C::H;
  constexpr int ROW = D + 8;                     // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) __bf16 sk[kTK][ROW];
  __shared__ __attribute__((aligned(16))) __bf16 sv[kTK][ROW];

  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int m0 = tile * kTK;
  const __bf16* kb = (const __bf16*)p.k + b * p.ks[0] + h * p.ks[1];
  const __bf16* vb = (const __bf16*)p.v + b * p.vs[0] + h * p.vs[1];
  const int64_t tix = ((int64_t)b * p.h_kv + h) * p.n_kt + tile;
  uint16_t* kp = (uint16_t*)p.kp + tix * (kTK * D);
  uint16_t* vp = (uint16_t*)p.vp + tix * (kTK * D);
  int ek, ev;
  head_range_exps(p.range, (int64_t)b * p.h_kv + h, &ek, &ev);

  // row-major copy of the tile into LDS; keys past n_kv are zero
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  for (int c = tid; c < kTK * CPR; c += 256) {
    const int key = c / CPR, ch = c % CPR;
    const int m = m0 + key;
    u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
    if (m < p.n_kv) {
      x = *reinterpret_cast<const u32x4*>(kb + (int64_t)m * p.ks[2] + ch * 8);
      y = *reinterpret_cast<const u32x4*>(vb + (int64_t)m * p.vs[2] + ch * 8);
    }
    *reinterpret_cast<u32x4*>(&sk[key][ch * 8]) = x;
    *reinterpret_cast<u32x4*>(&sv[key][ch * 8]) = y;
  }
  __syncthreads();

  // K' blocks: lane l of block (ks, blk) holds key 32*blk + l%32, pairs
  // 8*ks + 4*(l/32) + u, u = 0..3, rotated and scaled by 2^-ek, as
  // (x_r, x_{r+h}) fp16 pairs
  for (int it = tid; it < C::KBLK * 64; it += 256) {
    const int blk = it >> 6, lane = it & 63;
    const int key = 32 * (blk & 1) + (lane & 31);
    const int r0 = 8 * (blk >> 1) + 4 * (lane >> 5);
    const int m = m0 + key;
    u32x4 out;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x1 = (float)sk[key][r0 + u], x2 = (float)sk[key][H + r0 + u];
      float s, c;
      rope_sincos(m, p.win.phi[r0 + u], &s, &c);
      out[u] = pack_f16(__builtin_amdgcn_ldexpf(x1 * c - x2 * s, -ek),
                        __builtin_amdgcn_ldexpf(x2 * c + x1 * s, -ek));
    }
    *reinterpret_cast<u32x4*>(kp + blk_off(blk, lane)) = out;
  }
  // V blocks: lane l of block (bd, g) holds head-dim 32*bd + l%32 of keys
  // pv_key(g, l/32, j), j = 0..7, scaled by 2^-ev, fp16
  for (int it = tid; it < C::VBLK * 64; it += 256) {
    const int blk = it >> 6, lane = it & 63;
    const int bd = blk >> 2, g = blk & 3;
    const int dim = 32 * bd + (lane & 31), s = lane >> 5;
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 8; j += 2)
      out[j >> 1] = pack_f16(__builtin_amdgcn_ldexpf((float)sv[pv_key(g, s, j)][dim], -ev),
                             __builtin_amdgcn_ldexpf((float)sv[pv_key(g, s, j + 1)][dim], -ev));
    *reinterpret_cast<u32x4*>(vp + blk_off(blk, lane)) = out;
  }
}

template <int D, bool SPARSE, bool CAUSAL>
__global__ __launch_bounds__(PCfg<D>::THREADS, D == 64 ? 4 : 3) void prefill_bf16_kernel(const PrefillParams p) {
  using C = PCfg<D>;
  constexpr int H = C::H;
  constexpr int TILE = kTK * D;
  __shared__ __attribute__((aligned(16))) uint16_t lk[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t lq[C::WAVES][C::NKS * 512];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sh = lane >> 5, l32 = lane & 31;

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

  const __bf16* qbase = (const __bf16*)p.q + bb * p.qs[0] + hq * p.qs[1];
  const int64_t obase = bb * p.os[0] + hq * p.os[1];   // element offset of the output head
  const int64_t tix0 = ((int64_t)bb * p.n_kv_heads + kvh) * p.n_kt;
  const uint16_t* kpk = (const uint16_t*)p.kp + tix0 * TILE;
  const uint16_t* vpk = (const uint16_t*)p.vp + tix0 * TILE;
  int ek, ev;
  head_range_exps(p.range, (int64_t)bb * p.n_kv_heads + kvh, &ek, &ev);

  constexpr bool causal = CAUSAL;
  const int n_kv = p.n_kv;
  const int i0 = qb * C::BLOCK_ROWS;
  const int g_last = min(i0 + C::BLOCK_ROWS - 1, p.n_q - 1);
  const int w_first = i0 + wave * kRowsW;
  const int w_last = min(w_first + kRowsW - 1, p.n_q - 1);
  const bool wave_rows = w_first <= w_last;
  const int n_lo = p.q_pos0 + w_first, n_hi = p.q_pos0 + w_last;
  const int gn_lo = p.q_pos0 + i0, gn_hi = p.q_pos0 + g_last;
  const int qrow = min(w_first + l32, p.n_q - 1);
  const int npos = p.q_pos0 + qrow;
  const int w_lane = lane < H ? p.win.w[lane] : kWindowInf;

  // ---- query: load, rotate at its position, scale by softmax_scale *
  // log2(e) (scores in base-2 units) and by 2^ek (undoes the key scale), keep
  // as fp16 MFMA operand (lane l: query l%32, pairs 8ks + 4(l/32) + u as
  // (x_r, x_{r+h}) pairs), in registers and in a per-wave LDS copy (read at a
  // k-step chosen at run time).  If the wave's largest value reaches 2^14 the
  // operand carries 2^-eq, undone on the scores.
  uint16_t* qw_lds = &lq[wave][0];
  const __bf16* qrow_ptr = qbase + (int64_t)qrow * p.qs[2];
  f16x8 qop[C::Q_IN_LDS ? 1 : C::NKS];
  int eq;
  {
    const float cq = __builtin_amdgcn_ldexpf(p.scale_log2, ek);
    float qt[C::NKS][8];
    float qmax = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int r0 = 8 * ks + 4 * sh;
      const u32x2 a = *reinterpret_cast<const u32x2*>(qrow_ptr + r0);
      const u32x2 b = *reinterpret_cast<const u32x2*>(qrow_ptr + H + r0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x1 = (u & 1) ? bf16_hi(a[u >> 1]) : bf16_lo(a[u >> 1]);
        const float x2 = (u & 1) ? bf16_hi(b[u >> 1]) : bf16_lo(b[u >> 1]);
        float s, c;
        rope_sincos(npos, p.win.phi[r0 + u], &s, &c);
        qt[ks][2 * u] = (x1 * c - x2 * s) * cq;
        qt[ks][2 * u + 1] = (x2 * c + x1 * s) * cq;
        qmax = fmaxf(qmax, fmaxf(fabsf(qt[ks][2 * u]), fabsf(qt[ks][2 * u + 1])));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, o));
    eq = __builtin_amdgcn_readfirstlane(range_exp_of_float(qmax));
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      u32x4 packed;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        packed[u] = pack_f16(__builtin_amdgcn_ldexpf(qt[ks][2 * u], -eq),
                             __builtin_amdgcn_ldexpf(qt[ks][2 * u + 1], -eq));
      if constexpr (!C::Q_IN_LDS) qop[ks] = __builtin_bit_cast(f16x8, packed);
      *reinterpret_cast<u32x4*>(qw_lds + blk_off(ks, lane)) = packed;
    }
  }
  const float score_unscale = __builtin_amdgcn_ldexpf(1.0f, eq);   // scores carry 2^-eq

  f32x16 oacc[C::ND];
#pragma unroll
  for (int b = 0; b < C::ND; ++b) oacc[b] = f32x16{};
  float r_ref = 0.f, l_run = 0.f;   // reference (base 2) and running sum of the weights
  float raise_at = -INFINITY;       // kRaise once a visible key has set r_ref

  const int kv_end = causal ? min(n_kv, gn_hi + 1) : n_kv;
  const int n_kt = (kv_end + kTK - 1) / kTK;

  // ---- staging: direct global -> LDS copies (global_load_lds_dwordx4: 16
  // bytes per lane, lane l to byte 16 l of the destination, which is the
  // operand-block layout itself), one tile ahead: while a tile is worked from
  // one LDS buffer, the copies of the next visited tile fill the other and
  // are waited for at the end of the tile, before the barrier.  No staging
  // registers and no LDS store instructions.  Wave w copies K' blocks w + 8i
  // and V blocks w + 8i; a K' block of a k-step that the window drops for
  // every cell of the workgroup is not copied (its slot is never read).
  // First k-step any cell of the workgroup needs in key tile t (wave-uniform).
  auto stage_ks = [&](int t) -> int {
    const int m_lo = t * kTK;
    const int m_hi = min(m_lo + kTK - 1, n_kv - 1);
    int dmin = 0, dmax = 0;
    if (!span32(gn_lo, gn_hi, m_lo, m_hi, causal, &dmin, &dmax)) return C::NKS;
    return first_kstep(w_lane, dmin);
  };
  typedef __attribute__((address_space(3))) void lds_void;
  // copies of tile t into LDS slot `slot`: this wave's V blocks and K' blocks
  auto dma = [&](int t, int slot) {
    const uint16_t* ks = kpk + (int64_t)t * TILE;
    const uint16_t* vs = vpk + (int64_t)t * TILE;
    uint16_t* kd = &lk[slot][0];
    uint16_t* vd = &lv[slot][0];
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) {
      const int blk = wave + C::WAVES * i;
      if (C::VBLK % C::WAVES == 0 || blk < C::VBLK)
        __builtin_amdgcn_global_load_lds((const void*)(vs + blk_off(blk, lane)),
                                         (lds_void*)(vd + blk_off(blk, 0)), 16, 0, 0);
    }
    const int ks0 = stage_ks(t);
#pragma unroll
    for (int i = 0; i < C::KPW; ++i) {
      const int blk = wave + C::WAVES * i;
      if ((C::KBLK % C::WAVES == 0 || blk < C::KBLK) && (blk >> 1) >= ks0)
        __builtin_amdgcn_global_load_lds((const void*)(ks + blk_off(blk, lane)),
                                         (lds_void*)(kd + blk_off(blk, 0)), 16, 0, 0);
    }
  };

  // ---- key tiles visited, ascending.  Dense: 0 .. n_kt-1.  Block-sparse
  // (composition with a token-level selection): the tiles that some 64-row
  // query block of this workgroup selected, read 32 at a time from the
  // selection words (scalar loads, wave-uniform); a wave works a tile only
  // when its own query block selected it, and copies it to LDS either way.
  int cursor = -1;                 // dense: last tile handed out
  int sel_w = -1;                  // sparse: mask word being consumed
  uint32_t sel_rest = 0;           // sparse: union bits of word sel_w not yet handed out
  uint32_t sel_own = 0;            // sparse: this wave's bits of word sel_w
  const uint32_t* sel_row0 = nullptr;
  int n_sel_blk = 0, own_blk = 0;
  const int n_words = (n_kt + 31) >> 5;
  if constexpr (SPARSE) {
    const int qb0 = i0 / kSparseBlock;
    sel_row0 = p.sel + ((int64_t)(bb * p.h_q + hq) * p.n_sel_qb + qb0) * p.sel_words;
    n_sel_blk = min(C::BLOCK_ROWS / kSparseBlock, p.n_sel_qb - qb0);
    own_blk = (wave * kRowsW) / kSparseBlock;
  }
  auto next_tile = [&](int* t, bool* own) {
    if constexpr (!SPARSE) {
      ++cursor;
      *t = cursor < n_kt ? cursor : -1;
      *own = true;
    } else {
      while (sel_rest == 0) {
        if (++sel_w >= n_words) {
          *t = -1;
          *own = false;
          return;
        }
        const uint32_t valid = (n_kt - 32 * sel_w >= 32) ? 0xffffffffu : ((1u << (n_kt - 32 * sel_w)) - 1u);
        uint32_t u = 0, mine = 0;
        for (int j = 0; j < n_sel_blk; ++j) {
          const uint32_t word = __builtin_amdgcn_readfirstlane(sel_row0[(int64_t)j * p.sel_words + sel_w]);
          u |= word;
          if (j == own_blk) mine = word;
        }
        sel_rest = u & valid;
        sel_own = mine;
      }
      const int b = __builtin_ctz(sel_rest);
      sel_rest &= sel_rest - 1;
      *t = 32 * sel_w + b;
      *own = ((sel_own >> b) & 1u) != 0;
    }
  };

  // ---- prologue: K' buffers zeroed (a K' block the window prunes for the
  // whole workgroup is never copied, and is read only against a fully masked
  // query operand, which needs finite data), then the first tile in LDS
#pragma unroll
  for (int i = 0; i < (2 * TILE / 8 + C::THREADS - 1) / C::THREADS; ++i)
    if ((2 * TILE / 8) % C::THREADS == 0 || tid + C::THREADS * i < 2 * TILE / 8)
      reinterpret_cast<u32x4*>(&lk[0][0])[tid + C::THREADS * i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  int t = -1, t_next = -1, slot = 0;
  bool own = false, own_next = false;
  next_tile(&t, &own);
  if (t >= 0) dma(t, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  while (t >= 0) {
    next_tile(&t_next, &own_next);
    // copies of the next tile, issued at the top of the tile by every wave
    // (whether it works this tile or not).  Issued after the QK^T MFMAs
    // instead, they measured 2.5% slower at head_dim 128 and 0.5-1.8% slower
    // at head_dim 64; split between the two places, no faster.
    if (t_next >= 0) dma(t_next, slot ^ 1);

    const int m_lo = t * kTK;
    const int m_hi = min(m_lo + kTK - 1, n_kv - 1);
    int dmin = 0, dmax = 0;
    if (own && wave_rows && span32(n_lo, n_hi, m_lo, m_hi, causal, &dmin, &dmax)) {
      const int r_any = wave_pairs_below(w_lane, dmin);
      const int r_full = wave_pairs_below(w_lane, dmax);
      const int kbase_lane = m_lo + 4 * sh;
      const uint16_t* kt = &lk[slot][0];
      const uint16_t* vt = &lv[slot][0];
      // scores start from -r (in the operand's 2^-eq units)
      const float init = -r_ref * __builtin_amdgcn_ldexpf(1.0f, -eq);
      f32x16 sacc[2];
      // accumulators set to -r in place, so the first MFMA of each chain
      // reads and writes the same registers
      auto start = [&]() {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          sacc[0][v] = init;
          sacc[1][v] = init;
        }
      };

      // reset the cells of x beyond the window of partially windowed pair pp
      auto drop_cells = [&](f32x16 (&x)[2], int pp, float reset) {
        int thr_lo, thr_hi;
        drop_bounds(npos, p.win.w[pp], kbase_lane, causal, kTK, &thr_lo, &thr_hi);
        if constexpr (CAUSAL) {
          // causal: only keys too far back are beyond the window (one compare
          // per cell)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (32 * blk + acc_row(v) < thr_lo) x[blk][v] = reset;
        } else {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int ko = 32 * blk + acc_row(v);
              if (ko < thr_lo || ko > thr_hi) x[blk][v] = reset;
            }
        }
      };
      auto kop = [&](int ks, int blk) -> f16x8 {
        return *reinterpret_cast<const f16x8*>(kt + blk_off(2 * ks + blk, lane));
      };
      auto mfma = [](f16x8 a, f16x8 b, f32x16 c) -> f32x16 {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
      };

      // pairs kept for every cell: k-steps kk0..NKS-1.  k-step kk0 first
      // (from -r; head_dim 64: on top of the partial pairs), with its query
      // operand read from the LDS copy and the pairs below r_full (partial)
      // masked out; then the k-steps above it with the query operands from
      // the registers (head_dim 128: the LDS copy), from the top.  The K'
      // operands of the upper half of the k-steps are read before the
      // branches (a block of a pruned k-step holds stale data that is never
      // used), the lower half once the loop reaches it, so each MFMA waits
      // only for its own reads.  (r_full == H, every pair partial or pruned:
      // k-step NKS-1 with all its slots masked, which yields -r; its K' slot
      // holds finite data, as the K' buffers start zeroed)
      // The waves of a SIMD leave the barrier together and all start with
      // their QK^T MFMAs: the wave issuing them takes precedence over the
      // others' vector work until they are issued (measured 0.5-1.9% faster
      // than equal priority, same output).
      __builtin_amdgcn_s_setprio(1);
      const int kk0 = min(r_full >> 3, C::NKS - 1);
      {
        // (head_dim 64: no early reads, its register budget is 128)
        constexpr int HALF = D == 64 ? C::NKS : C::NKS / 2;
        f16x8 ka[C::NKS][2];
#pragma unroll
        for (int ks = C::NKS - 1; ks >= HALF; --ks) {
          ka[ks][0] = kop(ks, 0);
          ka[ks][1] = kop(ks, 1);
        }
        // query operand of k-step pp's pair alone (one-hot pair slot)
        auto pair_op = [&](int pp) -> f16x8 {
          const int ks = pp >> 3, uu = pp & 7;
          const uint32_t qd =
              *reinterpret_cast<const uint32_t*>(qw_lds + blk_off(ks, lane) + 2 * (uu & 3));
          const bool mine = sh == (uu >> 2);
          u32x4 bw;
#pragma unroll
          for (int d = 0; d < 4; ++d) bw[d] = (mine && d == (uu & 3)) ? qd : 0u;
          return __builtin_bit_cast(f16x8, bw);
        };
        {
          u32x4 bw = *reinterpret_cast<const u32x4*>(qw_lds + blk_off(kk0, lane));
          const int tau = r_full - 8 * kk0 - 4 * sh;   // slots below tau are partial
#pragma unroll
          for (int u = 0; u < 4; ++u) bw[u] = (u < tau) ? 0u : bw[u];
          const f16x8 bop = __builtin_bit_cast(f16x8, bw);
          if (D == 64 && r_any < r_full) {
            // partially windowed pairs [r_any, r_full) first, one pair per
            // MFMA, ascending, each followed by the reset of the cells beyond
            // its window to -r (windows grow with r, so what remains is
            // exactly the kept partial terms); then the masked k-step on top
            start();
            for (int pp = r_any; pp < r_full; ++pp) {
              const f16x8 bp = pair_op(pp);
              sacc[0] = mfma(kop(pp >> 3, 0), bp, sacc[0]);
              sacc[1] = mfma(kop(pp >> 3, 1), bp, sacc[1]);
              drop_cells(sacc, pp, init);
            }
            sacc[0] = mfma(kop(kk0, 0), bop, sacc[0]);
            sacc[1] = mfma(kop(kk0, 1), bop, sacc[1]);
          } else {
            start();
            sacc[0] = mfma(kop(kk0, 0), bop, sacc[0]);
            sacc[1] = mfma(kop(kk0, 1), bop, sacc[1]);
          }
        }
#pragma unroll
        for (int ks = C::NKS - 1; ks >= 1; --ks) {
          if (ks <= kk0) break;
          if (D == 64) {
            ka[ks][0] = kop(ks, 0);
            ka[ks][1] = kop(ks, 1);
          } else if (ks == HALF - 1) {
#pragma unroll
            for (int k2 = HALF - 1; k2 >= 1; --k2) {
              ka[k2][0] = kop(k2, 0);
              ka[k2][1] = kop(k2, 1);
            }
          }
          f16x8 qo;
          if constexpr (C::Q_IN_LDS)
            qo = *reinterpret_cast<const f16x8*>(qw_lds + blk_off(ks, lane));
          else
            qo = qop[ks];
          sacc[0] = mfma(ka[ks][0], qo, sacc[0]);
          sacc[1] = mfma(ka[ks][1], qo, sacc[1]);
        }
      }
      // head_dim 128: partially windowed pairs [r_any, r_full) one pair per
      // MFMA into a separate accumulator, ascending, each followed by the
      // reset to zero, then added (head_dim 64 handled them above, before the
      // kept k-steps, in the same accumulator: no zeroing and no final add,
      // which matters at its budget of 128 registers and vector-bound tile;
      // at head_dim 128 the separate accumulator measured faster)
      if (D != 64 && r_any < r_full) {
        f32x16 x[2] = {f32x16{}, f32x16{}};
        for (int pp = r_any; pp < r_full; ++pp) {
          const int ks = pp >> 3, uu = pp & 7;
          const f16x8 a0 = kop(ks, 0), a1 = kop(ks, 1);
          const uint32_t qd =
              *reinterpret_cast<const uint32_t*>(qw_lds + blk_off(ks, lane) + 2 * (uu & 3));
          const bool mine = sh == (uu >> 2);
          u32x4 bw;
#pragma unroll
          for (int d = 0; d < 4; ++d) bw[d] = (mine && d == (uu & 3)) ? qd : 0u;
          const f16x8 bop = __builtin_bit_cast(f16x8, bw);
          x[0] = mfma(a0, bop, x[0]);
          x[1] = mfma(a1, bop, x[1]);
          drop_cells(x, pp, 0.f);
        }
        sacc[0] += x[0];
        sacc[1] += x[1];
      }
      __builtin_amdgcn_s_setprio(0);
      // the query operand's power of two (only for queries reaching 2^14)
      if (eq != 0) {
        sacc[0] *= score_unscale;
        sacc[1] *= score_unscale;
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

      // online softmax on scores relative to r (base 2): raise r when a score
      // passes it by more than kRaise, or at the row's first visible key
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[blk][v]);
      mx = half_swap_max(mx);
      const bool raise = mx > raise_at;
      if (__any(raise)) {
        const float dr = raise ? mx - kRefLag : 0.f;
        // < 2^-8 where a running sum exists; a row's first raise multiplies
        // zeros (min keeps it finite for very negative first scores)
        const float alpha = fminf(exp2f(-dr), 1.f);
#pragma unroll
        for (int b = 0; b < C::ND; ++b) oacc[b] *= alpha;
        l_run *= alpha;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) sacc[blk] -= dr;
        r_ref += dr;
        raise_at = raise ? kRaise : raise_at;
      }
      float lsum = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // V operands of this key group first, so their LDS latency overlaps
        // the exponentials below
        f16x8 va[C::ND];
#pragma unroll
        for (int b = 0; b < C::ND; ++b)
          va[b] = *reinterpret_cast<const f16x8*>(vt + blk_off(4 * b + g, lane));
        u32x4 pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v0 = 8 * (g & 1) + 2 * i;
          const float e0 = __builtin_amdgcn_exp2f(sacc[g >> 1][v0]);
          const float e1 = __builtin_amdgcn_exp2f(sacc[g >> 1][v0 + 1]);
          pw[i] = pack_f16(e0, e1);
          // the normalizer sums the same rounded weights the PV product uses
          lsum = sum_f16x2(pw[i], lsum);
        }
        const f16x8 pop = __builtin_bit_cast(f16x8, pw);
#pragma unroll
        for (int b = 0; b < C::ND; ++b) oacc[b] = mfma(va[b], pop, oacc[b]);
      }
      l_run += lsum;
    }

    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next tile have landed
    __syncthreads();
    t = t_next;
    own = own_next;
    slot ^= 1;
  }

  // ---- epilogue: O = O^T * 2^ev / l
  const float l_tot = half_swap_sum(l_run);
  // a row without an attended key gives 0
  const float inv = l_tot > 0.f ? __builtin_amdgcn_ldexpf(1.f / l_tot, ev) : 0.f;
  const int row = w_first + l32;
  if (wave_rows && row <= w_last) {
    const int64_t orow = obase + (int64_t)row * p.os[2];
#pragma unroll
    for (int b = 0; b < C::ND; ++b)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * b + 8 * v4 + 4 * sh;
        const float o0 = oacc[b][4 * v4] * inv, o1 = oacc[b][4 * v4 + 1] * inv;
        const float o2 = oacc[b][4 * v4 + 2] * inv, o3 = oacc[b][4 * v4 + 3] * inv;
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>((float*)p.o + orow + d0) = f32x4{o0, o1, o2, o3};
        } else {
          u32x2 w;
          w[0] = pack_bf16(o0, o1);
          w[1] = pack_bf16(o2, o3);
          *reinterpret_cast<u32x2*>((__bf16*)p.o + orow + d0) = w;
        }
      }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, const PackParams& pk, int head_dim,
                               hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_qblk * p.h_q * p.batch;
  if (blocks <= 0) return hipSuccess;
  dim3 pgrid((unsigned)pk.n_kt, (unsigned)pk.h_kv, (unsigned)pk.batch);
  dim3 rgrid((unsigned)kRangeChunks, (unsigned)pk.h_kv, (unsigned)pk.batch);
  dim3 grid((unsigned)blocks);
#define ATW_PREFILL(DD)                                                                            \
  const dim3 block(PCfg<DD>::THREADS);                                                               \
  hipLaunchKernelGGL(range_kernel<DD>, rgrid, dim3(256), 0, stream, pk);                             \
  hipLaunchKernelGGL(pack_kv_kernel<DD>, pgrid, dim3(256), 0, stream, pk);                           \
  if (p.sel) {                                                                                       \
    if (p.causal) hipLaunchKernelGGL((prefill_bf16_kernel<DD, true, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((prefill_bf16_kernel<DD, true, false>), grid, block, 0, stream, p);      \
  } else {                                                                                           \
    if (p.causal) hipLaunchKernelGGL((prefill_bf16_kernel<DD, false, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((prefill_bf16_kernel<DD, false, false>), grid, block, 0, stream, p);     \
  }
  if (head_dim == 128) {
    ATW_PREFILL(128);
  } else if (head_dim == 64) {
    ATW_PREFILL(64);
  } else {
    return hipErrorInvalidValue;
  }
#undef ATW_PREFILL
  return hipGetLastError();
}

}  // namespace atw
