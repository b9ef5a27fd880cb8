// Host-side window planner: integer windows, pruned-term counts, tile plans.
//
// Definitions: "ATFlash — Per-RoPE-Wavelength Attention Windows", README,
// "The idea" (pair r turns by (n-m)*theta_r; its term is zero beyond the
// distance w_r = k*lambda_r; the reduction is input independent and known in
// closed form before running) and "Porting to something else" (per key tile,
// the prefix of pairs that is never needed).
#pragma once

#include <cstdint>

namespace atw {

constexpr int kMaxHeadDim = 256;
constexpr int64_t kUnbounded = int64_t(1) << 62;

// W_r = floor(k * 2*pi / theta_r), theta_r = base^(-2r/d), in IEEE double;
// kUnbounded when the window is off, k = +inf, or the value reaches 2^62.
void window_widths(int head_dim, double rope_base, double k_turns, bool window_on, int64_t* w);

// theta_r / (2*pi): turns per position of pair r.
void pair_turns_per_position(int head_dim, double rope_base, double* phi);

// RoPE frequencies of a model whose config rescales them ("Using the ports":
// window tables are built from the RoPE base, the head dim and rope_scaling).
enum RopeKind { kRopePlain = 0, kRopeLinear = 1, kRopeLlama3 = 2, kRopeTable = 3 };
struct RopeSpec {
  int kind = kRopePlain;
  double base = 10000.0;
  double factor = 1.0;                  // linear, llama3
  double low_freq_factor = 1.0;         // llama3
  double high_freq_factor = 4.0;        // llama3
  double original_max_position = 8192;  // llama3
  const double* theta = nullptr;        // table: theta_r for r < d/2
};

// theta_r of every pair (radians per position).  Plain: base^(-2r/d).
// Linear: the plain frequencies divided by factor.  Llama3: pairs whose plain
// wavelength is below original_max_position / high_freq_factor keep their
// frequency, pairs whose wavelength is above original_max_position /
// low_freq_factor are divided by factor, and in between the frequency is the
// blend (1 - s) * theta / factor + s * theta with
// s = (original_max_position / wavelength - low_freq_factor) /
//     (high_freq_factor - low_freq_factor).  Table: as given.
// Returns false, with a reason, unless every theta_r is finite, > 0 and
// non-increasing in r (the windows then grow with r).
bool rope_theta(const RopeSpec& spec, int head_dim, double* theta, const char** why);

// W_r = floor(k * 2*pi / theta_r) from given frequencies (same operations as
// window_widths, which it reproduces bit for bit for the plain frequencies).
void window_widths_theta(int h, const double* theta, double k_turns, bool window_on, int64_t* w);

// W_r from a caller's table: each entry >= 0 and non-decreasing in r
// (entries above kUnbounded are taken as kUnbounded); every W_r is kUnbounded
// when the window is off.  Returns false, with a reason, for a bad table.
bool explicit_widths(int h, const int64_t* table, bool window_on, int64_t* w, const char** why);

// Number of pairs whose window is shorter than delta (pairs pruned at that
// distance).  w is non-decreasing; h entries.
int first_retained_pair(const int64_t* w, int h, int64_t delta);

// Exact (pruned, total) pair-term counts per (batch, query head): query i at
// position q_pos0 + i, key j at position j, visible iff j <= position (causal)
// or always (non-causal).  Closed form: one arithmetic series per pair.
void pruned_terms(int64_t n_q, int64_t n_kv, int64_t q_pos0, int head_dim, const int64_t* w,
                  bool causal, int64_t* pruned, int64_t* total);

// pruned_terms restricted to a block-sparse key selection: query block qb
// (rows [qb * block, ...)) attends key block kb (keys [kb * block, ...)) iff
// bit kb % 32 of mask[qb * mask_words + kb / 32] is set.  Closed form per
// selected rectangle and pair.
void pruned_terms_blocks(int64_t n_q, int64_t n_kv, int64_t q_pos0, int head_dim, const int64_t* w,
                         bool causal, const uint32_t* mask, int64_t mask_words, int block,
                         int64_t* pruned, int64_t* total);

// Smallest and largest distance over the visible cells of the tile
// rows [n_lo, n_hi] x keys [m_lo, m_hi] (positions).  Returns false when the
// tile has no visible cell.
bool tile_distance_range(int64_t n_lo, int64_t n_hi, int64_t m_lo, int64_t m_hi, bool causal,
                         int64_t* dmin, int64_t* dmax);

// Tile plan (r_any, r_full) per (query tile, key tile); (-1, -1) if empty.
void tile_plan(int head_dim, const int64_t* w, int64_t n_q, int64_t n_kv, int64_t q_pos0,
               bool causal, int tile_q, int tile_k, int32_t* plan);

}  // namespace atw
