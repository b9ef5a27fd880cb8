// C ABI of libatw (declared in include/atw.h): argument checks, the window
// planner, and the kernel launches.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "atw.h"
#include "kernels.h"
#include "planner.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATW_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_window(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                 int max_dim) {
  if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > max_dim)
    return fail(ATW_EINVAL, "head_dim must be even and in 2..%d (got %d)", max_dim, head_dim);
  if (!(rope_base > 1.0) || std::isinf(rope_base))
    return fail(ATW_EINVAL, "rope_base must be a finite value > 1 (got %g)", rope_base);
  if (window_on && !(k_turns > 0.0))
    return fail(ATW_EINVAL, "k_turns must be > 0 when the window is on (got %g)", k_turns);
  return ATW_OK;
}

// Frequencies and integer windows of a RoPE descriptor.
struct RopeWindow {
  double theta[atw::kMaxHeadDim / 2];
  int64_t widths[atw::kMaxHeadDim / 2];
};

// theta_r of the descriptor, then W_r: the caller's table when it gives one
// (k is then not used), else floor(k * 2*pi / theta_r); every W_r is
// ATW_UNBOUNDED when the window is off.
int resolve_rope(const atw_rope* rope, int32_t head_dim, double k_turns, int32_t window_on,
                 int max_dim, RopeWindow* out) {
  if (rope == nullptr) return fail(ATW_EINVAL, "rope is NULL");
  if (rope->flags & ~ATW_ROPE_HAS_WIDTHS)
    return fail(ATW_EINVAL, "rope: unknown flags 0x%x", (unsigned)rope->flags);
  const int64_t* given = (rope->flags & ATW_ROPE_HAS_WIDTHS) ? rope->widths : nullptr;
  if ((rope->flags & ATW_ROPE_HAS_WIDTHS) && given == nullptr)
    return fail(ATW_EINVAL, "rope: ATW_ROPE_HAS_WIDTHS with a NULL widths table");
  if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > max_dim)
    return fail(ATW_EINVAL, "head_dim must be even and in 2..%d (got %d)", max_dim, head_dim);
  if (window_on && given == nullptr && !(k_turns > 0.0))
    return fail(ATW_EINVAL, "k_turns must be > 0 when the window is on (got %g)", k_turns);
  atw::RopeSpec spec;
  spec.kind = rope->kind;
  spec.base = rope->base;
  spec.factor = rope->factor;
  spec.low_freq_factor = rope->low_freq_factor;
  spec.high_freq_factor = rope->high_freq_factor;
  spec.original_max_position = rope->original_max_position;
  spec.theta = rope->theta;
  const char* why = "";
  if (!atw::rope_theta(spec, head_dim, out->theta, &why)) return fail(ATW_EINVAL, "rope: %s", why);
  if (given != nullptr) {
    if (!atw::explicit_widths(head_dim / 2, given, window_on != 0, out->widths, &why))
      return fail(ATW_EINVAL, "rope: %s", why);
  } else {
    atw::window_widths_theta(head_dim / 2, out->theta, k_turns, window_on != 0, out->widths);
  }
  return ATW_OK;
}

atw_rope plain_rope(double base) {
  atw_rope r{};
  r.kind = ATW_ROPE_PLAIN;
  r.base = base;
  return r;
}

// Kernel view of a resolved window: W_r clamped to INT32_MAX and turns per
// position theta_r / (2*pi).
void fill_window_rope(atw::WindowArgs* w, int head_dim, const RopeWindow& rw) {
  const double two_pi = 2.0 * 3.141592653589793;
  for (int r = 0; r < atw::kMaxPairs; ++r) {
    if (r < head_dim / 2) {
      w->w[r] = rw.widths[r] > (int64_t)atw::kWindowInf ? atw::kWindowInf : (int32_t)rw.widths[r];
      w->phi[r] = rw.theta[r] / two_pi;
    } else {
      w->w[r] = atw::kWindowInf;
      w->phi[r] = 0.0;
    }
  }
}

// Kernel view of the window: W_r clamped to INT32_MAX and turns per position.
void fill_window(atw::WindowArgs* w, int head_dim, double rope_base, double k_turns, bool on) {
  int64_t widths[atw::kMaxHeadDim / 2];
  atw::window_widths(head_dim, rope_base, k_turns, on, widths);
  double phi[atw::kMaxHeadDim / 2];
  atw::pair_turns_per_position(head_dim, rope_base, phi);
  for (int r = 0; r < atw::kMaxPairs; ++r) {
    if (r < head_dim / 2) {
      w->w[r] = widths[r] > (int64_t)atw::kWindowInf ? atw::kWindowInf : (int32_t)widths[r];
      w->phi[r] = phi[r];
    } else {
      w->w[r] = atw::kWindowInf;
      w->phi[r] = 0.0;
    }
  }
}

int check_heads(int32_t h_q, int32_t h_kv, const int32_t* map, int16_t* out) {
  if (h_q <= 0 || h_kv <= 0) return fail(ATW_EINVAL, "h_q and h_kv must be positive");
  if (h_q > atw::kMaxHeadsQ || h_kv > atw::kMaxHeadsQ)
    return fail(ATW_EUNSUPPORTED, "h_q and h_kv must be <= %d", atw::kMaxHeadsQ);
  if (map == nullptr) {
    if (h_q % h_kv != 0)
      return fail(ATW_EINVAL, "h_q (%d) must be a multiple of h_kv (%d) without a head map", h_q, h_kv);
    for (int h = 0; h < h_q; ++h) out[h] = (int16_t)(h / (h_q / h_kv));
  } else {
    for (int h = 0; h < h_q; ++h) {
      if (map[h] < 0 || map[h] >= h_kv)
        return fail(ATW_EINVAL, "kv_head_of_q[%d] = %d is outside [0, %d)", h, map[h], h_kv);
      out[h] = (int16_t)map[h];
    }
  }
  return ATW_OK;
}

int check_strides(const char* name, const int64_t* s, int n, int elem) {
  if (s == nullptr) return fail(ATW_EINVAL, "%s_strides is NULL", name);
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(ATW_EINVAL, "%s_strides[%d] is negative", name, i);
    if ((s[i] * elem) % 16 != 0)
      return fail(ATW_EUNSUPPORTED, "%s_strides[%d] = %lld is not a multiple of 16 bytes", name, i,
                  (long long)s[i]);
  }
  return ATW_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATW_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* atw_last_error(void) { return g_last_error.c_str(); }

const char* atw_version(void) { return "atw 0.3 (gfx950)"; }

int atw_window_widths(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                      int64_t* widths_out) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  if (widths_out == nullptr) return fail(ATW_EINVAL, "widths_out is NULL");
  atw::window_widths(head_dim, rope_base, k_turns, window_on != 0, widths_out);
  return ok();
}

int atw_pruned_terms(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim, double rope_base,
                     double k_turns, int32_t causal, int32_t window_on, int64_t* pruned,
                     int64_t* total) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  if (pruned == nullptr || total == nullptr) return fail(ATW_EINVAL, "pruned/total is NULL");
  if (n_q < 0 || n_kv < 0 || q_pos0 < 0) return fail(ATW_EINVAL, "n_q, n_kv, q_pos0 must be >= 0");
  if (n_q > (int64_t(1) << 40) || n_kv > (int64_t(1) << 40) || q_pos0 > (int64_t(1) << 40))
    return fail(ATW_EINVAL, "sizes above 2^40 are not supported");
  int64_t w[atw::kMaxHeadDim / 2];
  atw::window_widths(head_dim, rope_base, k_turns, window_on != 0, w);
  atw::pruned_terms(n_q, n_kv, q_pos0, head_dim, w, causal != 0, pruned, total);
  return ok();
}

int atw_rope_theta(const atw_rope* rope, int32_t head_dim, double* theta_out) {
  if (theta_out == nullptr) return fail(ATW_EINVAL, "theta_out is NULL");
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, 1.0, 0, atw::kMaxHeadDim, &rw)) return e;
  for (int r = 0; r < head_dim / 2; ++r) theta_out[r] = rw.theta[r];
  return ok();
}

int atw_window_widths_rope(const atw_rope* rope, int32_t head_dim, double k_turns,
                           int32_t window_on, int64_t* widths_out) {
  if (widths_out == nullptr) return fail(ATW_EINVAL, "widths_out is NULL");
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  for (int r = 0; r < head_dim / 2; ++r) widths_out[r] = rw.widths[r];
  return ok();
}

int atw_pruned_terms_rope(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim,
                          const atw_rope* rope, double k_turns, int32_t causal, int32_t window_on,
                          int64_t* pruned, int64_t* total) {
  if (pruned == nullptr || total == nullptr) return fail(ATW_EINVAL, "pruned/total is NULL");
  if (n_q < 0 || n_kv < 0 || q_pos0 < 0) return fail(ATW_EINVAL, "n_q, n_kv, q_pos0 must be >= 0");
  if (n_q > (int64_t(1) << 40) || n_kv > (int64_t(1) << 40) || q_pos0 > (int64_t(1) << 40))
    return fail(ATW_EINVAL, "sizes above 2^40 are not supported");
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  const int64_t* w = rw.widths;
  atw::pruned_terms(n_q, n_kv, q_pos0, head_dim, w, causal != 0, pruned, total);
  return ok();
}

int atw_window_plan(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                    int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t causal, int32_t tile_q,
                    int32_t tile_k, int32_t* plan_out) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  if (plan_out == nullptr) return fail(ATW_EINVAL, "plan_out is NULL");
  if (n_q < 0 || n_kv < 0 || q_pos0 < 0 || tile_q <= 0 || tile_k <= 0)
    return fail(ATW_EINVAL, "sizes must be >= 0 and tiles > 0");
  int64_t w[atw::kMaxHeadDim / 2];
  atw::window_widths(head_dim, rope_base, k_turns, window_on != 0, w);
  atw::tile_plan(head_dim, w, n_q, n_kv, q_pos0, causal != 0, tile_q, tile_k, plan_out);
  return ok();
}

int atw_window_plan_device(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                           int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t causal,
                           int32_t tile_q, int32_t tile_k, int32_t* plan_out, int64_t* pruned_out,
                           void* stream) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, 2 * atw::kMaxPairs)) return e;
  if (plan_out == nullptr || pruned_out == nullptr) return fail(ATW_EINVAL, "output is NULL");
  if (n_q < 0 || n_kv < 0 || q_pos0 < 0 || tile_q <= 0 || tile_k <= 0)
    return fail(ATW_EINVAL, "sizes must be >= 0 and tiles > 0");
  if (n_q * n_kv > (int64_t(1) << 40) || q_pos0 + n_q > (int64_t(1) << 30) ||
      n_kv > (int64_t(1) << 30))
    return fail(ATW_EINVAL, "n_q * n_kv must be <= 2^40 and positions < 2^30");
  atw::PlanParams p{};
  p.plan = plan_out;
  p.pruned = pruned_out;
  p.n_q = n_q;
  p.n_kv = n_kv;
  p.q_pos0 = q_pos0;
  p.causal = causal != 0;
  p.tile_q = tile_q;
  p.tile_k = tile_k;
  p.h = head_dim / 2;
  p.n_qt = (n_q + tile_q - 1) / tile_q;
  p.n_kt = (n_kv + tile_k - 1) / tile_k;
  fill_window(&p.win, head_dim, rope_base, k_turns, window_on != 0);
  return hip_status(atw::launch_plan(p, (hipStream_t)stream), "plan kernel launch");
}

}  // extern "C"

namespace {

int prefill_impl(const void* q, const void* k, const void* v, void* o, int32_t dtype, int64_t batch,
                 int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q, int32_t h_kv,
                 const int32_t* kv_head_of_q, int32_t head_dim, const int64_t* q_strides,
                 const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
                 const RopeWindow& rw, int32_t causal, int32_t window_on,
                 double softmax_scale, void* workspace, size_t workspace_bytes, void* stream,
                 const uint32_t* block_mask = nullptr, bool sparse = false) {
  if (head_dim != 64 && head_dim != 128)
    return fail(ATW_EUNSUPPORTED, "prefill supports head_dim 64 and 128 (got %d)", head_dim);
  // bf16 inputs with an fp32 output: the bf16 path, storing floats
  const bool out_f32 = dtype == ATW_BF16_F32OUT;
  if (out_f32) dtype = ATW_BF16;
  if (sparse) {
    if (dtype != ATW_BF16) return fail(ATW_EUNSUPPORTED, "block-sparse prefill supports dtype ATW_BF16 only");
    if (block_mask == nullptr && n_q > 0) return fail(ATW_EINVAL, "block_mask is NULL");
    if (reinterpret_cast<uintptr_t>(block_mask) % 4 != 0) return fail(ATW_EINVAL, "block_mask must be 4-byte aligned");
  }
  if (dtype != ATW_F32 && dtype != ATW_BF16) return fail(ATW_EUNSUPPORTED, "dtype must be ATW_F32 or ATW_BF16");
  if (batch <= 0 || n_q < 0 || q_pos0 < 0) return fail(ATW_EINVAL, "batch > 0, n_q >= 0, q_pos0 >= 0 required");
  if (n_kv < 1) return fail(ATW_EINVAL, "n_kv must be >= 1");
  if (q_pos0 + n_q > (int64_t(1) << 30) || n_kv > (int64_t(1) << 30))
    return fail(ATW_EUNSUPPORTED, "positions must be < 2^30");
  if (!std::isfinite(softmax_scale)) return fail(ATW_EINVAL, "softmax_scale must be finite");
  int16_t kvh[atw::kMaxHeadsQ];
  if (int e = check_heads(h_q, h_kv, kv_head_of_q, kvh)) return e;
  if (n_q == 0) return ok();   // nothing to compute; empty tensors may have NULL data
  if (!q || !k || !v || !o) return fail(ATW_EINVAL, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATW_EUNSUPPORTED, "q, k, v and o must be 16-byte aligned");
  const int elem = dtype == ATW_BF16 ? 2 : 4;
  if (int e = check_strides("q", q_strides, 3, elem)) return e;
  if (int e = check_strides("k", k_strides, 3, elem)) return e;
  if (int e = check_strides("v", v_strides, 3, elem)) return e;
  if (int e = check_strides("o", o_strides, 3, out_f32 ? 4 : elem)) return e;
  const int64_t rows = dtype == ATW_BF16 ? atw::prefill_bf16_block_rows(head_dim) : atw::kPrefillBlockRows;
  const int64_t n_qblk = (n_q + rows - 1) / rows;
  if (n_qblk * h_q * batch >= (int64_t(1) << 31)) return fail(ATW_EUNSUPPORTED, "grid too large");
  if (batch > 65535) return fail(ATW_EUNSUPPORTED, "batch must be <= 65535");
  const size_t need = atw_prefill_workspace_bytes(dtype, batch, h_kv, n_kv, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATW_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (need > 0 && !aligned16(workspace)) return fail(ATW_EUNSUPPORTED, "workspace must be 16-byte aligned");

  atw::PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = q_strides[i];
    p.ks[i] = k_strides[i];
    p.vs[i] = v_strides[i];
    p.os[i] = o_strides[i];
  }
  p.batch = (int32_t)batch;
  p.n_q = (int32_t)n_q;
  p.n_kv = (int32_t)n_kv;
  p.q_pos0 = (int32_t)q_pos0;
  p.h_q = h_q;
  p.causal = causal != 0;
  p.n_qblk = (int32_t)n_qblk;
  p.n_kv_heads = h_kv;
  p.out_f32 = out_f32 ? 1 : 0;
  const double scale = softmax_scale > 0 ? softmax_scale : 1.0 / std::sqrt((double)head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  // query heads grouped by kv head: workgroups of one kv head share an XCD
  int n = 0;
  for (int kv = 0; kv < h_kv; ++kv) {
    p.kv_first[kv] = (int16_t)n;
    for (int h = 0; h < h_q; ++h)
      if (kvh[h] == kv) p.qh_of_kv[n++] = (int16_t)h;
  }
  p.kv_first[h_kv] = (int16_t)n;
  fill_window_rope(&p.win, head_dim, rw);
  if (sparse) {
    p.sel = block_mask;
    p.n_sel_qb = (int32_t)((n_q + atw::kSparseBlock - 1) / atw::kSparseBlock);
    p.sel_words = (int32_t)atw_block_mask_words(n_kv);
  }
  if (dtype == ATW_F32)
    return hip_status(atw::launch_prefill_f32(p, head_dim, (hipStream_t)stream), "prefill launch");

  atw::PackParams pk{};
  pk.k = k;
  pk.v = v;
  const size_t tiles = atw::prefill_tile_bytes(batch, h_kv, n_kv, head_dim);
  pk.kp = workspace;
  pk.vp = static_cast<char*>(workspace) + tiles;
  pk.range = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 2 * tiles);
  for (int i = 0; i < 3; ++i) {
    pk.ks[i] = k_strides[i];
    pk.vs[i] = v_strides[i];
  }
  pk.n_kv = (int32_t)n_kv;
  pk.n_kt = (int32_t)((n_kv + atw::kPrefillTileK - 1) / atw::kPrefillTileK);
  pk.h_kv = h_kv;
  pk.batch = (int32_t)batch;
  pk.win = p.win;
  p.kp = pk.kp;
  p.vp = pk.vp;
  p.range = pk.range;
  p.n_kt = pk.n_kt;
  return hip_status(atw::launch_prefill_bf16(p, pk, head_dim, (hipStream_t)stream), "prefill launch");
}

}  // namespace

extern "C" {

int atw_prefill(const void* q, const void* k, const void* v, void* o, int32_t dtype, int64_t batch,
                int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q, int32_t h_kv,
                const int32_t* kv_head_of_q, int32_t head_dim, const int64_t* q_strides,
                const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
                double rope_base, double k_turns, int32_t causal, int32_t window_on,
                double softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  const atw_rope rope = plain_rope(rope_base);
  RopeWindow rw;
  if (int e = resolve_rope(&rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return prefill_impl(q, k, v, o, dtype, batch, n_q, n_kv, q_pos0, h_q, h_kv, kv_head_of_q, head_dim,
                      q_strides, k_strides, v_strides, o_strides, rw, causal, window_on,
                      softmax_scale, workspace, workspace_bytes, stream);
}

int atw_prefill_rope(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                     int64_t batch, int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q,
                     int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                     const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                     int32_t window_on, double softmax_scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return prefill_impl(q, k, v, o, dtype, batch, n_q, n_kv, q_pos0, h_q, h_kv, kv_head_of_q, head_dim,
                      q_strides, k_strides, v_strides, o_strides, rw, causal, window_on,
                      softmax_scale, workspace, workspace_bytes, stream);
}

int atw_prefill_sparse(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                       int64_t batch, int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q,
                       int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                       const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                       const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                       int32_t window_on, double softmax_scale, const uint32_t* block_mask,
                       void* workspace, size_t workspace_bytes, void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return prefill_impl(q, k, v, o, dtype, batch, n_q, n_kv, q_pos0, h_q, h_kv, kv_head_of_q, head_dim,
                      q_strides, k_strides, v_strides, o_strides, rw, causal, window_on,
                      softmax_scale, workspace, workspace_bytes, stream, block_mask, true);
}

int64_t atw_block_mask_words(int64_t n_kv) {
  if (n_kv <= 0) return 0;
  const int64_t n_kb = (n_kv + atw::kSparseBlock - 1) / atw::kSparseBlock;
  return (n_kb + 31) / 32;
}

int atw_pruned_terms_sparse(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim,
                            const atw_rope* rope, double k_turns, int32_t causal, int32_t window_on,
                            const uint32_t* block_mask, int64_t* pruned, int64_t* total) {
  if (pruned == nullptr || total == nullptr) return fail(ATW_EINVAL, "pruned/total is NULL");
  if (n_q < 0 || n_kv < 0 || q_pos0 < 0) return fail(ATW_EINVAL, "n_q, n_kv, q_pos0 must be >= 0");
  if (n_q > (int64_t(1) << 40) || n_kv > (int64_t(1) << 40) || q_pos0 > (int64_t(1) << 40))
    return fail(ATW_EINVAL, "sizes above 2^40 are not supported");
  if (block_mask == nullptr && n_q > 0 && n_kv > 0) return fail(ATW_EINVAL, "block_mask is NULL");
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  const int64_t* w = rw.widths;
  if (n_q == 0 || n_kv == 0) {
    *pruned = 0;
    *total = 0;
    return ok();
  }
  atw::pruned_terms_blocks(n_q, n_kv, q_pos0, head_dim, w, causal != 0, block_mask,
                           atw_block_mask_words(n_kv), atw::kSparseBlock, pruned, total);
  return ok();
}

size_t atw_prefill_workspace_bytes(int32_t dtype, int64_t batch, int32_t h_kv, int64_t n_kv,
                                   int32_t head_dim) {
  if ((dtype != ATW_BF16 && dtype != ATW_BF16_F32OUT) || batch <= 0 || h_kv <= 0 || n_kv <= 0 ||
      head_dim <= 0)
    return 0;
  return atw::prefill_pack_bytes(batch, h_kv, n_kv, head_dim);
}

size_t atw_decode_workspace_bytes(int64_t batch, int32_t h_q, int32_t head_dim, int32_t num_splits) {
  if (batch <= 0 || h_q <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return (size_t)batch * (size_t)h_q * (size_t)num_splits * (size_t)(head_dim + 4) * sizeof(float);
}

namespace {

// Shared body of atw_decode (row-layout K cache) and atw_decode_banded.
int decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                int64_t batch, int32_t q_len, int64_t q_tok_stride, int64_t o_tok_stride,
                const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                const int64_t* o_strides, const RopeWindow& rw, int32_t causal,
                int32_t window_on, double softmax_scale, int32_t num_splits, void* workspace,
                size_t workspace_bytes, void* stream, bool banded, const uint32_t* block_mask = nullptr,
                int64_t mask_words = 0, bool sparse = false) {
  if (head_dim != 64 && head_dim != 128)
    return fail(ATW_EUNSUPPORTED, "decode supports head_dim 64 and 128 (got %d)", head_dim);
  if (dtype != ATW_BF16 && dtype != ATW_BF16_F32OUT)
    return fail(ATW_EUNSUPPORTED, "decode supports dtype ATW_BF16 and ATW_BF16_F32OUT only");
  const bool out_f32 = dtype == ATW_BF16_F32OUT;
  if (batch <= 0 || batch > atw::kMaxDecodeBatch)
    return fail(ATW_EUNSUPPORTED, "batch must be in 1..%d", atw::kMaxDecodeBatch);
  if (num_splits <= 0 || num_splits > atw::kMaxDecodeSplits)
    return fail(ATW_EINVAL, "num_splits must be in 1..%d", atw::kMaxDecodeSplits);
  if (!std::isfinite(softmax_scale)) return fail(ATW_EINVAL, "softmax_scale must be finite");
  if (kv_len == nullptr || q_pos == nullptr) return fail(ATW_EINVAL, "kv_len and q_pos must be non-NULL");
  for (int64_t b = 0; b < batch; ++b) {
    if (kv_len[b] < 1 || kv_len[b] > (int64_t(1) << 30))
      return fail(ATW_EINVAL, "kv_len[%lld] = %lld must be in 1..2^30", (long long)b, (long long)kv_len[b]);
    if (q_pos[b] < 0 || q_pos[b] >= (int64_t(1) << 30))
      return fail(ATW_EINVAL, "q_pos[%lld] out of range", (long long)b);
    if (causal && q_pos[b] + q_len - 1 < kv_len[b] - 1)
      return fail(ATW_EINVAL, "causal decode needs q_pos[%lld] + q_len - 1 >= kv_len - 1", (long long)b);
    if (q_pos[b] + q_len - 1 >= (int64_t(1) << 30))
      return fail(ATW_EINVAL, "q_pos[%lld] + q_len - 1 out of range", (long long)b);
  }
  if (sparse) {
    if (block_mask == nullptr) return fail(ATW_EINVAL, "block_mask is NULL");
    if (reinterpret_cast<uintptr_t>(block_mask) % 4 != 0) return fail(ATW_EINVAL, "block_mask must be 4-byte aligned");
    if (q_len != 1) return fail(ATW_EUNSUPPORTED, "block-sparse decode takes one query token per sequence");
    int64_t max_len = 0;
    for (int64_t b = 0; b < batch; ++b) max_len = std::max(max_len, kv_len[b]);
    if (mask_words < atw_block_mask_words(max_len) || mask_words > (int64_t(1) << 24))
      return fail(ATW_EINVAL, "mask_words must be >= atw_block_mask_words(max kv_len) (%lld)",
                  (long long)atw_block_mask_words(max_len));
  }
  int16_t kvh[atw::kMaxHeadsQ];
  if (int e = check_heads(h_q, h_kv, kv_head_of_q, kvh)) return e;
  if (!q || !k_cache || !v_cache || !o) return fail(ATW_EINVAL, "q, k_cache, v_cache and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATW_EUNSUPPORTED, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (int e = check_strides("q", q_strides, 2, 2)) return e;
  if (int e = check_strides("k", k_strides, 3, 2)) return e;
  if (int e = check_strides("v", v_strides, 3, 2)) return e;
  if (o_strides == nullptr || o_strides[0] < 0 || o_strides[1] < 0)
    return fail(ATW_EINVAL, "o_strides must be non-NULL and non-negative");
  const size_t need = (size_t)q_len * atw_decode_workspace_bytes(batch, h_q, head_dim, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATW_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(ATW_EUNSUPPORTED, "workspace must be 16-byte aligned");

  atw::DecodeParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o = o;
  p.out_f32 = out_f32 ? 1 : 0;
  p.ws = static_cast<float*>(workspace);
  p.qs[0] = q_strides[0];
  p.qs[1] = q_strides[1];
  p.qs[2] = q_tok_stride;
  p.os[0] = o_strides[0];
  p.os[1] = o_strides[1];
  p.os[2] = o_tok_stride;
  p.q_len = q_len;
  for (int i = 0; i < 3; ++i) {
    p.ks[i] = k_strides[i];
    p.vs[i] = v_strides[i];
  }
  p.batch = (int32_t)batch;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.splits = num_splits;
  p.causal = causal != 0;
  const double scale = softmax_scale > 0 ? softmax_scale : 1.0 / std::sqrt((double)head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  for (int64_t b = 0; b < batch; ++b) {
    p.kv_len[b] = (int32_t)kv_len[b];
    p.q_pos[b] = (int32_t)q_pos[b];
  }
  // group query heads by kv head; a kv head may serve at most 16 query heads
  int n = 0;
  for (int kv = 0; kv < h_kv; ++kv) {
    p.kv_first[kv] = (int16_t)n;
    int cnt = 0;
    for (int h = 0; h < h_q; ++h)
      if (kvh[h] == kv) {
        p.qh_of_kv[n++] = (int16_t)h;
        ++cnt;
      }
    if (cnt * q_len > 16)
      return fail(ATW_EUNSUPPORTED, "decode supports at most 16 (query head, token) columns per kv head");
  }
  p.kv_first[h_kv] = (int16_t)n;
  p.group = h_q / h_kv;
  // kv head kv serves query heads kv * group .. kv * group + group - 1, in
  // order: the kernels then compute a column's query head instead of reading
  // it from the tables
  p.heads_in_order = h_q % h_kv == 0 ? 1 : 0;   // (an explicit map may give h_q < h_kv)
  for (int i = 0; i < h_q && p.heads_in_order; ++i)
    if (p.qh_of_kv[i] != i || kvh[i] != i / p.group) p.heads_in_order = 0;
  if (sparse) {
    p.sel = block_mask;
    p.sel_words = (int32_t)mask_words;
  }
  fill_window_rope(&p.win, head_dim, rw);
  return hip_status(atw::launch_decode(p, head_dim, banded, (hipStream_t)stream), "decode launch");
}

}  // namespace

int atw_decode(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
               int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
               int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
               const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
               const int64_t* o_strides, double rope_base, double k_turns, int32_t causal,
               int32_t window_on, double softmax_scale, int32_t num_splits, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  const atw_rope rope = plain_rope(rope_base);
  RopeWindow rw;
  if (int e = resolve_rope(&rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return decode_impl(q, k_cache, v_cache, o, dtype, batch, 1, 0, 0, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                     head_dim, q_strides, k_strides, v_strides, o_strides, rw,
                     causal, window_on, softmax_scale, num_splits, workspace, workspace_bytes,
                     stream, false);
}

int atw_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                       int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                       int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                       const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                       const int64_t* o_strides, double rope_base, double k_turns, int32_t causal,
                       int32_t window_on, double softmax_scale, int32_t num_splits, void* stream) {
  const size_t need = atw_decode_workspace_bytes(batch, h_q, head_dim, num_splits);
  if (need > atw::kDecodeScratchBytes)
    return fail(ATW_EWORKSPACE,
                "atw_decode_noalloc: the split partials need %zu bytes, more than its %zu-byte device "
                "array (use fewer splits or atw_decode with a workspace)",
                need, (size_t)atw::kDecodeScratchBytes);
  void* scratch = nullptr;
  if (int e = hip_status(atw::decode_scratch(&scratch), "decode scratch lookup")) return e;
  return atw_decode(q, k_cache, v_cache, o, dtype, batch, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                    head_dim, q_strides, k_strides, v_strides, o_strides, rope_base, k_turns, causal,
                    window_on, softmax_scale, num_splits, scratch, atw::kDecodeScratchBytes, stream);
}

size_t atw_decode_noalloc_max_bytes(void) { return atw::kDecodeScratchBytes; }

int atw_decode_rope(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                    int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                    int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                    const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                    const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                    int32_t window_on, double softmax_scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return decode_impl(q, k_cache, v_cache, o, dtype, batch, 1, 0, 0, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                     head_dim, q_strides, k_strides, v_strides, o_strides, rw,
                     causal, window_on, softmax_scale, num_splits, workspace, workspace_bytes,
                     stream, false);
}

int atw_decode_banded(const void* q, const void* k_bands, const void* v_cache, void* o,
                      int32_t dtype, int64_t batch, const int64_t* kv_len, const int64_t* q_pos,
                      int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                      const int64_t* q_strides, const int64_t* k_strides,
                      const int64_t* v_strides, const int64_t* o_strides, double rope_base,
                      double k_turns, int32_t causal, int32_t window_on, double softmax_scale,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (int e = check_window(head_dim, rope_base, k_turns, window_on, atw::kMaxHeadDim)) return e;
  const atw_rope rope = plain_rope(rope_base);
  RopeWindow rw;
  if (int e = resolve_rope(&rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return decode_impl(q, k_bands, v_cache, o, dtype, batch, 1, 0, 0, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                     head_dim, q_strides, k_strides, v_strides, o_strides, rw,
                     causal, window_on, softmax_scale, num_splits, workspace, workspace_bytes,
                     stream, true);
}

int atw_decode_banded_rope(const void* q, const void* k_bands, const void* v_cache, void* o,
                           int32_t dtype, int64_t batch, const int64_t* kv_len,
                           const int64_t* q_pos, int32_t h_q, int32_t h_kv,
                           const int32_t* kv_head_of_q, int32_t head_dim, const int64_t* q_strides,
                           const int64_t* k_strides, const int64_t* v_strides,
                           const int64_t* o_strides, const atw_rope* rope, double k_turns,
                           int32_t causal, int32_t window_on, double softmax_scale,
                           int32_t num_splits, void* workspace, size_t workspace_bytes,
                           void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return decode_impl(q, k_bands, v_cache, o, dtype, batch, 1, 0, 0, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                     head_dim, q_strides, k_strides, v_strides, o_strides, rw,
                     causal, window_on, softmax_scale, num_splits, workspace, workspace_bytes,
                     stream, true);
}

int atw_decode_sparse(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                      int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                      int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                      const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                      const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                      int32_t window_on, double softmax_scale, int32_t num_splits,
                      const uint32_t* block_mask, int64_t mask_words, int32_t k_banded,
                      void* workspace, size_t workspace_bytes, void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  return decode_impl(q, k_cache, v_cache, o, dtype, batch, 1, 0, 0, kv_len, q_pos, h_q, h_kv, kv_head_of_q,
                     head_dim, q_strides, k_strides, v_strides, o_strides, rw, causal,
                     window_on, softmax_scale, num_splits, workspace, workspace_bytes, stream,
                     k_banded != 0, block_mask, mask_words, true);
}

size_t atw_decode_multi_workspace_bytes(int64_t batch, int32_t q_len, int32_t h_q, int32_t head_dim,
                                        int32_t num_splits) {
  if (q_len <= 0) return 0;
  return (size_t)q_len * atw_decode_workspace_bytes(batch, h_q, head_dim, num_splits);
}

int atw_decode_multi(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                     int64_t batch, int32_t q_len, const int64_t* kv_len, const int64_t* q_pos,
                     int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                     const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, int32_t k_banded, const atw_rope* rope,
                     double k_turns, int32_t window_on, double softmax_scale, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  RopeWindow rw;
  if (int e = resolve_rope(rope, head_dim, k_turns, window_on, atw::kMaxHeadDim, &rw)) return e;
  if (q_len < 1 || q_len > 16) return fail(ATW_EINVAL, "q_len must be in 1..16 (got %d)", q_len);
  if (q_strides == nullptr || o_strides == nullptr) return fail(ATW_EINVAL, "q_strides / o_strides is NULL");
  if (q_strides[2] < 0 || o_strides[2] < 0 || (q_strides[2] * 2) % 16 != 0)
    return fail(ATW_EINVAL, "token strides must be non-negative (q: a multiple of 16 bytes)");
  int16_t kvh[atw::kMaxHeadsQ];
  if (int e = check_heads(h_q, h_kv, kv_head_of_q, kvh)) return e;
  int gmax = 0;
  for (int kv = 0; kv < h_kv; ++kv) {
    int cnt = 0;
    for (int h = 0; h < h_q; ++h) cnt += kvh[h] == kv;
    gmax = cnt > gmax ? cnt : gmax;
  }
  if (gmax > 16) return fail(ATW_EUNSUPPORTED, "at most 16 query heads per kv head");
  const size_t need = atw_decode_multi_workspace_bytes(batch, q_len, h_q, head_dim, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATW_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (batch <= 0 || batch > atw::kMaxDecodeBatch)
    return fail(ATW_EUNSUPPORTED, "batch must be in 1..%d", atw::kMaxDecodeBatch);
  if (kv_len == nullptr || q_pos == nullptr) return fail(ATW_EINVAL, "kv_len and q_pos must be non-NULL");
  for (int64_t bb = 0; bb < batch; ++bb) {
    if (kv_len[bb] < 1 || kv_len[bb] > (int64_t(1) << 30))
      return fail(ATW_EINVAL, "kv_len[%lld] = %lld must be in 1..2^30", (long long)bb, (long long)kv_len[bb]);
    if (q_pos[bb] < 0 || q_pos[bb] + q_len - 1 >= (int64_t(1) << 30))
      return fail(ATW_EINVAL, "q_pos[%lld] out of range", (long long)bb);
    if (q_pos[bb] + q_len - 1 < kv_len[bb] - 1)
      return fail(ATW_EINVAL, "q_pos[%lld] + q_len - 1 >= kv_len - 1 is required", (long long)bb);
  }
  // the tokens go through the kernel in groups of at most 16 / gmax, one
  // launch per group (each launch streams the caches once)
  const int per = 16 / (gmax > 0 ? gmax : 1);
  int64_t pos[atw::kMaxDecodeBatch], kvl[atw::kMaxDecodeBatch];
  for (int t0 = 0; t0 < q_len; t0 += per) {
    const int n = q_len - t0 < per ? q_len - t0 : per;
    // the group's tokens see keys up to the position of its last token
    for (int64_t bb = 0; bb < batch; ++bb) {
      pos[bb] = q_pos[bb] + t0;
      kvl[bb] = kv_len[bb] < pos[bb] + n ? kv_len[bb] : pos[bb] + n;
    }
    const void* qg = static_cast<const char*>(q) + (int64_t)t0 * q_strides[2] * 2;
    void* og = static_cast<char*>(o) + (int64_t)t0 * o_strides[2] * (dtype == ATW_BF16_F32OUT ? 4 : 2);
    if (int e = decode_impl(qg, k_cache, v_cache, og, dtype, batch, n, q_strides[2], o_strides[2], kvl,
                            pos, h_q, h_kv, kv_head_of_q, head_dim, q_strides, k_strides, v_strides,
                            o_strides, rw, 1, window_on, softmax_scale, num_splits,
                            workspace, workspace_bytes, stream, k_banded != 0))
      return e;
  }
  return ok();
}

int atw_kcache_band(const void* k_rows, void* k_bands, int32_t dtype, int64_t batch, int32_t h_kv,
                    int32_t head_dim, int64_t t0, int64_t n_tokens, const int64_t* row_strides,
                    const int64_t* band_strides, void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(ATW_EUNSUPPORTED, "banding supports head_dim 64 and 128 (got %d)", head_dim);
  if (dtype != ATW_BF16) return fail(ATW_EUNSUPPORTED, "banding supports dtype ATW_BF16 only");
  if (batch < 1 || batch > 65535) return fail(ATW_EINVAL, "batch must be in 1..65535");
  if (h_kv < 1 || h_kv > 65535) return fail(ATW_EINVAL, "h_kv must be in 1..65535");
  if (t0 < 0 || n_tokens < 0 || t0 + n_tokens > (int64_t(1) << 30))
    return fail(ATW_EINVAL, "token range [t0, t0 + n_tokens) must lie in [0, 2^30)");
  if (n_tokens == 0) return ok();
  if (!k_rows || !k_bands) return fail(ATW_EINVAL, "k_rows and k_bands must be non-NULL");
  if (!aligned16(k_rows) || !aligned16(k_bands))
    return fail(ATW_EUNSUPPORTED, "k_rows and k_bands must be 16-byte aligned");
  if (int e = check_strides("row", row_strides, 3, 2)) return e;
  if (int e = check_strides("band", band_strides, 3, 2)) return e;
  atw::BandParams p{};
  p.rows = k_rows;
  p.bands = k_bands;
  for (int i = 0; i < 3; ++i) {
    p.rs[i] = row_strides[i];
    p.bs[i] = band_strides[i];
  }
  p.t0 = t0;
  p.n = n_tokens;
  p.batch = (int32_t)batch;
  p.h_kv = h_kv;
  return hip_status(atw::launch_kcache_band(p, head_dim, (hipStream_t)stream), "banding launch");
}

}  // extern "C"
