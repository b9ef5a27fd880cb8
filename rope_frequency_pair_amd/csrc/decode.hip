// Windowed split-KV decode and its combine pass for gfx950 (MI355X).
//
// Method: "ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
// idea": for a key at distance delta from the query, the pairs whose window
// is shorter than delta contribute nothing, so that prefix of the pre-RoPE
// key row is not loaded; the rest is rotated as it is loaded.  The split-KV
// partition and the merge of per-split (max, sum, output) partials are the
// standard online-softmax merge; the window does not change them.
//
// Work layout (CDNA4 design):
//  * one workgroup = one wave = one (sequence, kv head, split); the columns
//    of S^T = K' Q'^T (v_mfma_f32_16x16x32_bf16) are the query heads that read
//    this kv head (up to 16), so every key is loaded once for all of them;
//  * all query heads of a decode step sit at one position, so the window of
//    a cell depends on the key alone: the staging lane of a key zeroes the
//    pairs of that key beyond their window (and skips loading pair chunks
//    that are entirely beyond it), so the window is exact per key with no
//    extra MFMA work; whole k-steps pruned for a tile are skipped;
//  * key tiles of 32 keys; a lane owns one 8-pair chunk of every 8th key
//    (16th for d = 64), so its RoPE angle advances by a constant per round
//    (rotation recurrence, re-anchored exactly every 64 rounds);
//  * the next tile's K chunks and V rows are loaded into registers while the
//    current tile is computed from LDS; V stays row-major in LDS and is read
//    into the PV operand with the transposing LDS read;
//  * about 180 VGPRs and 20 KB of LDS per wave: 8 waves per CU, each with a
//    16 KB tile in flight;
//  * the cache streams (row-layout K, V) are read with non-temporal loads,
//    which stream markedly faster from HBM on this GPU (a plain streaming
//    read reaches ~7 TB/s with them, ~6.2 TB/s without); the banded K is read
//    with ordinary loads because each of its lines is covered by two load
//    instructions that the cache merges;
//  * the combine pass reads every split's (max, sum) at once, one split per
//    thread, instead of walking the splits serially.
#include "device_common.h"
#include "kernels.h"

namespace atw {
namespace {

constexpr int kTK = 32;              // keys per tile
constexpr int kReanchorRounds = 64;
constexpr float kRescaleLog2 = 8.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8 bytes addressed by lanes i/4, i/4+4, i/4+8, i/4+12 (in that order).
__device__ __forceinline__ v4i16 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<void*>(p));
}

template <int D>
struct DCfg {
  static constexpr int H = D / 2;
  static constexpr int NCH = H / 8;                 // 8-pair chunks per key
  static constexpr int KPR = 64 / NCH;              // keys staged per round (8 or 16)
  static constexpr int ROUNDS = kTK / KPR;          // staging rounds per tile
  static constexpr int KROW = D + 8;                // K' row (elements), pairs interleaved
  // V rows padded to a stride of 24 or 56 dwords mod 64: the transposing reads
  // of two 16-lane groups (8 consecutive rows) then use disjoint banks
  static constexpr int VROW = D == 128 ? 176 : 112;
  static constexpr int NVT = kTK * D * 2 / 16 / 64; // 16-byte V chunks per lane per tile
  static constexpr int NKS = D / 32;                // QK^T k-steps (16 pairs each)
  static constexpr int ND = D / 16;                 // 16-wide head-dim blocks
};

// Key range of one split.  The splits of a sequence carry equal byte cost:
// a key costs its V row plus the K bands it needs (banded cache: band c is
// fetched for the key iff its longest-window pair, 8c+7, is kept at the key's
// distance; row cache: every line of the row is fetched), in units of 32
// bytes, so with the window on and a banded cache the far splits, which need
// fewer bands, cover more keys.  Otherwise every key costs the same and the
// splits are equal.  Boundaries are multiples of 4 keys (one 128-byte line of
// a band) except the sequence end.
template <int D, bool BANDED>
__device__ void split_range(int kv_len, int qpos, bool causal, int splits, int split,
                            const int32_t* w, int* k_begin, int* k_end) {
  constexpr int NB = D / 16;
  auto cost_below = [&](int x) -> int64_t {     // cost of keys [0, x)
    int64_t c = (int64_t)(2 * D * 2 / 32) * x;  // V row: 2*D bytes
    if (!BANDED) return c + (int64_t)NB * x;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t wb = w[8 * b + 7];
      const int64_t lo = max((int64_t)0, (int64_t)qpos - wb);
      const int64_t hi = causal ? (int64_t)x : min((int64_t)x, (int64_t)qpos + wb + 1);
      c += max((int64_t)0, hi - lo);
    }
    return c;
  };
  const int64_t total = cost_below(kv_len);
  auto bound = [&](int s) -> int {
    if (s >= splits) return kv_len;
    const int64_t target = total * s;
    int lo = 0, hi = kv_len;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (cost_below(mid) * splits >= target) hi = mid; else lo = mid + 1;
    }
    return lo & ~3;
  };
  *k_begin = bound(split);
  *k_end = bound(split + 1);
}

// Block-sparse selection: the range of selected key blocks split `split` of
// `splits` takes (splits carry equal numbers of selected blocks).  row holds
// n_words mask words; blocks at or beyond nb are ignored.  Wave-wide: lanes
// read 64 words at a time, count bits, and a prefix scan over lanes finds
// the word and bit of the split's first block.  Returns the number of blocks
// and the position (word, bit) of the first.
__device__ __forceinline__ uint32_t valid_bits(int word, int nb) {
  const int rest = nb - 32 * word;
  return rest >= 32 ? 0xffffffffu : (rest <= 0 ? 0u : ((1u << rest) - 1u));
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ void sparse_split(const uint32_t* row, int n_words, int nb, int splits, int split,
                             int* first_word, int* first_bit, int* count) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int base = 0; base < n_words; base += 64) {
    const int wi = base + lane;
    const uint32_t w = wi < n_words ? row[wi] & valid_bits(wi, nb) : 0u;
    total += wave_sum_i32(__popc(w));
  }
  const int lo = (int)((int64_t)total * split / splits);
  const int hi = (int)((int64_t)total * (split + 1) / splits);
  *count = hi - lo;
  *first_word = n_words;
  *first_bit = 0;
  if (hi <= lo) return;
  int before = 0;
  for (int base = 0; base < n_words; base += 64) {
    const int wi = base + lane;
    const uint32_t w = wi < n_words ? row[wi] & valid_bits(wi, nb) : 0u;
    const int c = __popc(w);
    int incl = c;                                   // inclusive prefix over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int excl = incl - c;
    const bool here = lo >= before + excl && lo < before + incl;
    const uint64_t hit = __ballot(here);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      // the (lo - before - excl)-th set bit of this lane's word
      uint32_t rest = w;
      for (int k = lo - before - excl; k > 0 && rest; --k) rest &= rest - 1u;
      const int bit = rest ? __builtin_ctz(rest) : 0;
      *first_word = __shfl(wi, src);
      *first_bit = __shfl(bit, src);
      return;
    }
    before += __shfl(incl, 63);
  }
}

template <int D>
struct DSmem {
  __bf16 k[kTK][DCfg<D>::KROW];
  __bf16 v[kTK][DCfg<D>::VROW];
};

// BANDED: K cache stored as [batch, h_kv, h/8 bands, L, 16] (band c holds, per
// key, dims [8c, 8c+8) then [h+8c, h+8c+8)); ks[2] is the band stride and
// the token stride is 16.  A 128-byte line then holds one band of 4 keys,
// so a band the window prunes for those keys is not fetched at all.
// Otherwise K is [batch, h_kv, L, d] with ks[2] the token stride.
// MULTI: q_len > 1 query tokens per sequence at consecutive positions q_pos,
// q_pos + 1, ... (draft tokens of speculative / multi-token decoding), causal.
// The MFMA columns are (token, query head) pairs, token-major.  K' is staged
// with the window of token 0, the nearest one (distances grow with the token
// index, so token 0 keeps the most pairs); a tile in which some key has a pair
// whose window ends between the distances of token 0 and of the last token is
// recomputed token by token from the rotated values kept in registers, each
// lane keeping its own token's scores.  Keys after a token's position are
// masked out of that token's column.
template <int D, bool BANDED, bool MULTI, bool SPARSE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_split_kernel(const DecodeParams p) {
  using C = DCfg<D>;
  constexpr int H = C::H;
  __shared__ DSmem<D> sm;

  const int lane = threadIdx.x, l16 = lane & 15, grp4 = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int kv_len = p.kv_len[b];
  const int qpos = p.q_pos[b];
  const bool causal = p.causal != 0;
  int k_begin = 0, k_end = kv_len;
  // SPARSE: this split's selected key blocks, walked 32 at a time
  const uint32_t* sel_row = nullptr;
  int sel_word = 0, sel_left = 0;
  uint32_t sel_bits = 0;
  const int n_blocks = (kv_len + kSparseBlock - 1) / kSparseBlock;
  if constexpr (SPARSE) {
    sel_row = p.sel + ((int64_t)b * p.h_kv + kvh) * p.sel_words;
    int first_bit = 0;
    sparse_split(sel_row, min(p.sel_words, (n_blocks + 31) / 32), n_blocks, p.splits, split, &sel_word,
                 &first_bit, &sel_left);
    sel_word = __builtin_amdgcn_readfirstlane(sel_word);
    first_bit = __builtin_amdgcn_readfirstlane(first_bit);
    sel_left = __builtin_amdgcn_readfirstlane(sel_left);
    if (sel_left > 0)
      sel_bits = __builtin_amdgcn_readfirstlane(sel_row[sel_word]) & valid_bits(sel_word, n_blocks) &
                 (0xffffffffu << first_bit);
  } else {
    split_range<D, BANDED>(kv_len, qpos, causal, p.splits, split, p.win.w, &k_begin, &k_end);
  }

  const int g0 = p.kv_first[kvh], G = p.kv_first[kvh + 1] - g0;
  const int w_lane = lane < H ? p.win.w[lane] : kWindowInf;

  const __bf16* kbase = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* vbase = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];

  // query operand (B of 16x16x32): column l16 = the l16-th query head of this
  // kv head (MULTI: token l16 / G, head l16 % G), contraction slots 8*grp4.. of
  // k-step ks = pairs 16ks + 4grp4 + 0..3
  const int q_len = MULTI ? p.q_len : 1;
  const bool col_valid = l16 < G * q_len;
  const int tok = (MULTI && col_valid) ? l16 / G : 0;
  const int col_qh = col_valid ? p.qh_of_kv[g0 + (MULTI ? l16 % G : l16)] : 0;
  bf16x8 qop[C::NKS];
  {
    const bool valid = col_valid;
    const int qh = col_qh;
    const int tpos = qpos + tok;
    const __bf16* qrow = (const __bf16*)p.q + b * p.qs[0] + qh * p.qs[1] + tok * p.qs[2];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int r0 = 16 * ks + 4 * grp4;
      u32x4 packed = u32x4{0, 0, 0, 0};
      if (valid) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(qrow + r0);
        const u32x2 c2 = *reinterpret_cast<const u32x2*>(qrow + H + r0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x1 = (u & 1) ? bf16_hi(a[u >> 1]) : bf16_lo(a[u >> 1]);
          const float x2 = (u & 1) ? bf16_hi(c2[u >> 1]) : bf16_lo(c2[u >> 1]);
          float s, c;
          rope_sincos(tpos, p.win.phi[r0 + u], &s, &c);
          packed[u] = pack_bf16(x1 * c - x2 * s, x2 * c + x1 * s);
        }
      }
      qop[ks] = __builtin_bit_cast(bf16x8, packed);
    }
  }

  f32x4 oacc[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // K staging: lane = (key offset kj, pair chunk kc); its keys are kj, kj+KPR, ...
  // (banded: consecutive lanes take consecutive keys of one band)
  const int kj = BANDED ? lane % C::KPR : lane / C::NCH;
  const int kc = BANDED ? lane / C::KPR : lane % C::NCH;
  // RoPE step of one round (KPR keys) for the lane's 8 pairs
  float st_c[8], st_s[8], rc[8], rs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rope_sincos(C::KPR, p.win.phi[kc * 8 + e], &st_s[e], &st_c[e]);
  // windows of the lane's 8 pairs: pair kc*8+e is dropped for a key iff dist > W
  int wch[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wch[e] = p.win.w[kc * 8 + e];

  u32x4 kreg[C::ROUNDS][2];
  u32x4 vreg[C::NVT];
  const int n_tiles = (k_end - k_begin + kTK - 1) / kTK;

  auto key_dist = [&](int m) -> int {
    const int d = qpos - m;
    return (causal || d >= 0) ? d : -d;
  };

  auto load_tile = [&](int m0) {
#pragma unroll
    for (int i = 0; i < C::ROUNDS; ++i) {
      const int m = m0 + C::KPR * i + kj;
      // the chunk is needed iff its last (longest-window) pair is kept at this key
      if (m < k_end && key_dist(m) <= wch[7]) {
        if constexpr (BANDED) {
          const __bf16* src = kbase + (int64_t)kc * p.ks[2] + (int64_t)m * 16;
          // a lane's two loads are the halves of its key's 32 bytes, so each
          // load instruction covers every other 16 bytes of the band's lines:
          // ordinary loads, so the cache merges the two into one fetch
          kreg[i][0] = *reinterpret_cast<const u32x4*>(src);
          kreg[i][1] = *reinterpret_cast<const u32x4*>(src + 8);
        } else {
          const __bf16* src = kbase + (int64_t)m * p.ks[2] + kc * 8;
          // whole lines of the row per instruction: streamed
          kreg[i][0] = load_stream(src);
          kreg[i][1] = load_stream(src + H);
        }
      } else {
        kreg[i][0] = u32x4{0, 0, 0, 0};
        kreg[i][1] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVT; ++i) {
      const int task = lane + 64 * i;
      const int key = task / (D / 8), ch = task % (D / 8);
      const int m = m0 + key;
      if (m < k_end)
        vreg[i] = load_stream(vbase + (int64_t)m * p.vs[2] + ch * 8);
      else
        vreg[i] = u32x4{0, 0, 0, 0};
    }
  };

  int round_ix = 0;   // staging rounds done so far (drives the recurrence)
  // MULTI: rotated, packed K' pairs of the staged tile (not yet windowed), and
  // whether some key of the tile has a pair kept for token 0 but not for the
  // last token
  uint32_t rot[MULTI ? C::ROUNDS : 1][8];
  bool nonuni = false;
  auto store_tile = [&](int m0) {
    nonuni = false;
#pragma unroll
    for (int i = 0; i < C::ROUNDS; ++i) {
      const int m = m0 + C::KPR * i + kj;
      // exact angles every kReanchorRounds rounds, and (sparse) at the start
      // of every selected block, after which keys are no longer consecutive
      const bool anchor = SPARSE ? (i == 0 && (m0 & (kSparseBlock - 1)) == 0)
                                 : (round_ix % kReanchorRounds == 0);
      if (anchor) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_sincos(m, p.win.phi[kc * 8 + e], &rs[e], &rc[e]);
      }
      const int dist = key_dist(m);
      u32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wa = kreg[i][0][e >> 1], wb = kreg[i][1][e >> 1];
        const float x1 = (e & 1) ? bf16_hi(wa) : bf16_lo(wa);
        const float x2 = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
        uint32_t pk = pack_bf16(x1 * rc[e] - x2 * rs[e], x2 * rc[e] + x1 * rs[e]);
        if constexpr (MULTI) {
          rot[i][e] = pk;
          nonuni = nonuni || (dist <= wch[e] && dist + q_len - 1 > wch[e]);
        }
        pk = dist > wch[e] ? 0u : pk;             // pair beyond its window at this key
        if (e < 4) o0[e] = pk; else o1[e - 4] = pk;
      }
      __bf16* dst = &sm.k[C::KPR * i + kj][16 * kc];
      reinterpret_cast<u32x4*>(dst)[0] = o0;
      reinterpret_cast<u32x4*>(dst)[1] = o1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = rc[e], s = rs[e];
        rc[e] = c * st_c[e] - s * st_s[e];
        rs[e] = s * st_c[e] + c * st_s[e];
      }
      ++round_ix;
    }
#pragma unroll
    for (int i = 0; i < C::NVT; ++i) {
      const int task = lane + 64 * i;
      const int key = task / (D / 8), ch = task % (D / 8);
      *reinterpret_cast<u32x4*>(&sm.v[key][ch * 8]) = vreg[i];
    }
  };

  // MULTI: rewrite the staged K' tile windowed for token j (distance + j)
  auto rewrite_k = [&](int m0, int j) {
#pragma unroll
    for (int i = 0; i < C::ROUNDS; ++i) {
      const int m = m0 + C::KPR * i + kj;
      const int dist = key_dist(m) + j;
      u32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pk = dist > wch[e] ? 0u : rot[MULTI ? i : 0][e];
        if (e < 4) o0[e] = pk; else o1[e - 4] = pk;
      }
      __bf16* dst = &sm.k[C::KPR * i + kj][16 * kc];
      reinterpret_cast<u32x4*>(dst)[0] = o0;
      reinterpret_cast<u32x4*>(dst)[1] = o1;
    }
  };

  // tiles visited: dense, the split's consecutive tiles; sparse, the two
  // 32-key halves of each selected block (the second only if it holds keys)
  int t_dense = -1;
  int half = 1, cur_block = -1;
  auto next_tile = [&]() -> int {
    if constexpr (!SPARSE) {
      ++t_dense;
      return t_dense < n_tiles ? k_begin + t_dense * kTK : -1;
    } else {
      if (half == 0 && kSparseBlock * cur_block + kTK < kv_len) {
        half = 1;
        return kSparseBlock * cur_block + kTK;
      }
      if (sel_left == 0) return -1;
      while (sel_bits == 0) {
        ++sel_word;
        sel_bits = __builtin_amdgcn_readfirstlane(sel_row[sel_word]) & valid_bits(sel_word, n_blocks);
      }
      cur_block = 32 * sel_word + __builtin_ctz(sel_bits);
      sel_bits &= sel_bits - 1u;
      --sel_left;
      half = 0;
      return kSparseBlock * cur_block;
    }
  };

  int m_cur = next_tile();
  if (m_cur >= 0) load_tile(m_cur);

  while (m_cur >= 0) {
    store_tile(m_cur);
    __syncthreads();
    const int m_next = next_tile();
    if (m_next >= 0) load_tile(m_next);

    const int m_lo = m_cur;
    const int m_hi = min(m_lo + kTK - 1, k_end - 1);
    int64_t dmin = 0, dmax = 0;
    tile_distance_range(qpos, qpos, m_lo, m_hi, causal, &dmin, &dmax);
    const int r_any = wave_pairs_below(w_lane, dmin);   // pairs below: zero for every key

    // S^T = K' Q'^T over the k-steps that hold some kept pair
    auto qk = [&](f32x4 (&s)[2]) {
      s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        if (16 * ks + 16 <= r_any) continue;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[16 * blk + l16][32 * ks + 8 * grp4]);
          s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[ks], s[blk], 0, 0, 0);
        }
      }
    };
    f32x4 sacc[2];
    qk(sacc);
    if constexpr (MULTI) {
      if (__any(nonuni)) {
        // some pair's window ends between the tokens' distances in this tile:
        // recompute for each later token from the rotated values
        for (int j = 1; j < q_len; ++j) {
          __syncthreads();
          rewrite_k(m_cur, j);
          __syncthreads();
          f32x4 sj[2];
          qk(sj);
          if (tok == j) {
            sacc[0] = sj[0];
            sacc[1] = sj[1];
          }
        }
      }
      // keys after a token's position (the later draft tokens' own keys)
      if (m_hi > qpos) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (m_lo + 16 * blk + 4 * grp4 + v > qpos + tok) sacc[blk][v] = -INFINITY;
      }
    }

    // keys past the end of the split
    if (m_lo + kTK > k_end) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (m_lo + 16 * blk + 4 * grp4 + v >= k_end) sacc[blk][v] = -INFINITY;
    }

    // online softmax per query-head column (lanes l16, l16+16, l16+32, l16+48)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sacc[blk][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool grow = (m_new - m_run) * p.scale_log2 > kRescaleLog2;
    if (__any(grow)) {
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f((m_run - m_new) * p.scale_log2);
#pragma unroll
      for (int i = 0; i < C::ND; ++i) oacc[i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float mb = (m_run == -INFINITY) ? 0.f : m_run * p.scale_log2;
    // P^T operand: slots 8*grp4 + e = keys 4grp4 + e (e < 4) and 16 + 4grp4 + e - 4
    u32x4 pw;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i >> 1][2 * (i & 1)], p.scale_log2, -mb));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i >> 1][2 * (i & 1) + 1], p.scale_log2, -mb));
      pw[i] = pack_bf16(e0, e1);
      lsum = sum_bf16x2(pw[i], lsum);      // normalizer of the rounded weights
    }
    l_run += lsum;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);

    // O^T += V^T P^T: transposing reads give lane l four keys of dim 16bd + l16
#pragma unroll
    for (int bd = 0; bd < C::ND; ++bd) {
      const __bf16* base = &sm.v[4 * grp4 + ((lane & 15) >> 2)][16 * bd + 4 * (lane & 3)];
      const v4i16 lo = lds_read_tr16(base);
      const v4i16 hi = lds_read_tr16(base + 16 * C::VROW);
      const bf16x8 a = __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      oacc[bd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop, oacc[bd], 0, 0, 0);
    }
    __syncthreads();   // LDS reads done before the next store
    m_cur = m_next;
  }

  // partial result of this split: [m (raw score units), l, -, -, o[D]] per query head
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = half_swap_sum(l_tot);
  if (col_valid) {
    const int qh = col_qh;
    float* w = p.ws + ((((int64_t)b * q_len + tok) * p.h_q + qh) * p.splits + split) * (D + 4);
    if (grp4 == 0) {
      w[0] = m_run;
      w[1] = l_tot;
    }
#pragma unroll
    for (int bd = 0; bd < C::ND; ++bd)
      *reinterpret_cast<f32x4*>(w + 4 + 16 * bd + 4 * grp4) = oacc[bd];
  }
}

// Merge the splits of one (sequence, query head): standard online-softmax
// merge of (max, sum, unnormalised output) partials.  The splits' maxima and
// weights are read by all threads at once (one split per thread, strided),
// so the merge costs a few dependent memory round trips, not one per split.
// The weighted sum of the outputs is spread over G = kCombineThreads / D
// groups of D threads (group g takes splits g, g + G, ...), whose partial
// sums meet in LDS: with hundreds of splits and a handful of blocks per
// call (one sequence, few heads) a single group would walk the splits one
// memory round trip after another.
constexpr int kCombineThreads = 512;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const DecodeParams p) {
  constexpr int T = kCombineThreads, NW = T / 64, G = T / D;
  __shared__ float weight[kMaxDecodeSplits];
  __shared__ float part[NW];
  __shared__ float gsum[G - 1][D];
  // blockIdx.y = sequence * q_len + token
  const int qh = blockIdx.x, bt = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int d = tid % D, g = tid / D;
  const int b = bt / p.q_len, tok = bt % p.q_len;
  const int S = p.splits;
  const float* w = p.ws + ((int64_t)bt * p.h_q + qh) * S * (D + 4);
  auto block_reduce = [&](float x, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float y = __shfl_xor(x, o);
      x = is_max ? fmaxf(x, y) : x + y;
    }
    if (lane == 0) part[wv] = x;
    __syncthreads();
    x = part[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) x = is_max ? fmaxf(x, part[i]) : x + part[i];
    __syncthreads();
    return x;
  };
  float m = -INFINITY;
  for (int s = tid; s < S; s += T) m = fmaxf(m, w[s * (D + 4)]);
  m = block_reduce(m, true);
  float l = 0.f;
  for (int s = tid; s < S; s += T) {
    const float ms = w[s * (D + 4)];
    const float a = (ms == -INFINITY) ? 0.f : exp2f((ms - m) * p.scale_log2);
    weight[s] = a;
    l += a * w[s * (D + 4) + 1];
  }
  l = block_reduce(l, false);   // its barriers also publish weight[]
  float acc = 0.f;
#pragma unroll 8
  for (int s = g; s < S; s += G) acc += weight[s] * w[s * (D + 4) + 4 + d];
  if (g > 0) gsum[g - 1][d] = acc;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < G - 1; ++i) acc += gsum[i][d];
    __bf16* o = (__bf16*)p.o + b * p.os[0] + qh * p.os[1] + tok * p.os[2];
    o[d] = (__bf16)(l > 0.f ? acc / l : 0.f);   // no attended key: 0
  }
}

// Row-layout K cache -> pair-banded K cache, for tokens [t0, t0 + n) of every
// (batch, kv head): one thread copies the two 16-byte halves of one band of
// one key.
template <int D>
__global__ __launch_bounds__(256) void kcache_band_kernel(const BandParams p) {
  constexpr int NB = D / 16;                        // bands (8 pairs each)
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.n * NB) return;
  const int64_t m = p.t0 + idx / NB;
  const int c = (int)(idx % NB);
  const int h = blockIdx.y, b = blockIdx.z;
  const __bf16* src = (const __bf16*)p.rows + b * p.rs[0] + h * p.rs[1] + m * p.rs[2] + 8 * c;
  __bf16* dst = (__bf16*)p.bands + b * p.bs[0] + h * p.bs[1] + c * p.bs[2] + m * 16;
  reinterpret_cast<u32x4*>(dst)[0] = *reinterpret_cast<const u32x4*>(src);
  reinterpret_cast<u32x4*>(dst)[1] = *reinterpret_cast<const u32x4*>(src + D / 2);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, bool banded, hipStream_t stream) {
  dim3 grid((unsigned)p.splits, (unsigned)p.h_kv, (unsigned)p.batch);
  dim3 cgrid((unsigned)p.h_q, (unsigned)(p.batch * p.q_len));
  const bool multi = p.q_len > 1;
  const bool sparse = p.sel != nullptr;
  if (multi && sparse) return hipErrorInvalidValue;
#define ATW_DECODE_SPLIT(DD, BB, MM, SS) \
  hipLaunchKernelGGL((decode_split_kernel<DD, BB, MM, SS>), grid, dim3(64), 0, stream, p)
#define ATW_DECODE_ALL(DD)                                                         \
  if (sparse) {                                                                    \
    if (banded) ATW_DECODE_SPLIT(DD, true, false, true);                           \
    else ATW_DECODE_SPLIT(DD, false, false, true);                                 \
  } else if (multi) {                                                              \
    if (banded) ATW_DECODE_SPLIT(DD, true, true, false);                           \
    else ATW_DECODE_SPLIT(DD, false, true, false);                                 \
  } else {                                                                         \
    if (banded) ATW_DECODE_SPLIT(DD, true, false, false);                          \
    else ATW_DECODE_SPLIT(DD, false, false, false);                                \
  }                                                                                \
  hipLaunchKernelGGL((decode_combine_kernel<DD>), cgrid, dim3(kCombineThreads), 0, stream, p)
  if (head_dim == 128) {
    ATW_DECODE_ALL(128);
  } else if (head_dim == 64) {
    ATW_DECODE_ALL(64);
  } else {
    return hipErrorInvalidValue;
  }
#undef ATW_DECODE_ALL
#undef ATW_DECODE_SPLIT
  return hipGetLastError();
}

hipError_t launch_kcache_band(const BandParams& p, int head_dim, hipStream_t stream) {
  const int64_t work = p.n * (head_dim / 16);
  if (work <= 0) return hipSuccess;
  dim3 grid((unsigned)((work + 255) / 256), (unsigned)p.h_kv, (unsigned)p.batch);
  if (head_dim == 128)
    hipLaunchKernelGGL(kcache_band_kernel<128>, grid, dim3(256), 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(kcache_band_kernel<64>, grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace atw
