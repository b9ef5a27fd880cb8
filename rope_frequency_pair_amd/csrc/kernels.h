// Kernel parameter blocks and launchers (host side of the HIP kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace atw {

constexpr int kMaxHeadsQ = 256;
constexpr int kMaxDecodeBatch = 256;

// Prefill: one workgroup = consecutive query rows of one query head, 32 per
// wave; key tiles of 64.  fp32: 8 waves (256 rows).
constexpr int kPrefillBlockRows = 256;
// bf16 prefill: waves (32 query rows each) per workgroup by head_dim
constexpr int prefill_bf16_waves(int head_dim) { return head_dim == 128 ? 12 : 8; }
constexpr int prefill_bf16_block_rows(int head_dim) { return 32 * prefill_bf16_waves(head_dim); }
constexpr int kPrefillTileK = 64;

// Range pass of the bf16 prefill: chunks of keys per (batch, kv head) whose
// largest |k| and |v| are recorded (2 x uint32 bf16 magnitude bits each).
constexpr int kRangeChunks = 32;

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const void* kp;                        // bf16: packed K' / V tiles (pack_kv_kernel), fp16
  const void* vp;
  const uint32_t* range;                 // bf16: [batch, h_kv, kRangeChunks, 2] (range_kernel)
  int64_t qs[3], ks[3], vs[3], os[3];   // element strides (batch, head, token)
  int32_t batch, n_q, n_kv, q_pos0;
  int32_t h_q, causal, n_qblk, n_kv_heads;
  int32_t n_kt;                          // packed key tiles per (batch, kv head)
  int32_t out_f32;                       // bf16: 1 = fp32 output (o is float)
  float scale_log2;                      // softmax scale * log2(e)
  // Block-sparse key selection (nullptr: every key).  Bit kb % 32 of word
  // kb / 32 of row ((b * h_q + hq) * n_sel_qb + qb), rows of sel_words words:
  // query block qb (64 rows) attends key block kb (64 keys).
  const uint32_t* sel;
  int32_t sel_words, n_sel_qb;
  int16_t qh_of_kv[kMaxHeadsQ];          // query heads grouped by kv head (kv-major)
  int16_t kv_first[kMaxHeadsQ + 1];      // start of each kv head's group in qh_of_kv
  WindowArgs win;
};

// Decode: split-KV over the key axis, then a combine pass.
constexpr int kDecodeTileK = 64;
constexpr int kSparseBlock = 64;         // query rows / keys per block of a block-sparse selection
constexpr int kMaxDecodeSplits = 1024;

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* ws;                             // [batch, q_len, h_q, splits, head_dim + 4]
  int64_t qs[3], ks[3], vs[3], os[3];   // q / o: (batch, head, token) element strides
  int32_t batch, h_q, h_kv, splits;
  int32_t causal, group, q_len;         // group = query heads per kv head; q_len tokens per sequence
  int32_t heads_in_order;               // 1: kv head k serves query heads k * group + 0 .. group - 1
  // Block-sparse key selection (nullptr: every key): bit kb % 32 of word
  // kb / 32 of row (b * h_kv + kvh), rows of sel_words words: the sequence's
  // kv head attends key block kb (64 keys).
  const uint32_t* sel;
  int32_t sel_words;
  int32_t out_f32;                       // 1 = fp32 output (o is float)
  float scale_log2;
  int32_t kv_len[kMaxDecodeBatch];
  int32_t q_pos[kMaxDecodeBatch];
  int16_t qh_of_kv[kMaxHeadsQ];          // query heads grouped by kv head (kv-major)
  int16_t kv_first[kMaxHeadsQ + 1];      // start of each kv head's group in qh_of_kv
  WindowArgs win;
};

// Packing of K (rotated) and V into matrix-core operand order, 64-key tiles:
// kp/vp [batch, h_kv, n_kt, 64 * head_dim] fp16 (scaled by the range
// exponents of their (batch, kv head)).
struct PackParams {
  const void* k;
  const void* v;
  void* kp;
  void* vp;
  uint32_t* range;                       // [batch, h_kv, kRangeChunks, 2]
  int64_t ks[3], vs[3];
  int32_t n_kv, n_kt, h_kv, batch;
  WindowArgs win;
};

// Workspace of a bf16 prefill: packed K' tiles, packed V tiles (each
// prefill_tile_bytes), then the range pass's chunk maxima.
inline size_t prefill_tile_bytes(int64_t batch, int64_t h_kv, int64_t n_kv, int64_t head_dim) {
  const int64_t n_kt = (n_kv + kPrefillTileK - 1) / kPrefillTileK;
  return (size_t)(batch * h_kv * n_kt * kPrefillTileK * head_dim * 2);
}
inline size_t prefill_pack_bytes(int64_t batch, int64_t h_kv, int64_t n_kv, int64_t head_dim) {
  return 2 * prefill_tile_bytes(batch, h_kv, n_kv, head_dim) +
         (size_t)(batch * h_kv * kRangeChunks * 2 * 4);
}

struct BandParams {
  const void* rows;
  void* bands;
  int64_t rs[3], bs[3];                  // (batch, head, token) / (batch, head, band) strides
  int64_t t0, n;                         // tokens [t0, t0 + n)
  int32_t batch, h_kv;
};

struct PlanParams {
  int32_t* plan;
  int64_t* pruned;
  int64_t n_q, n_kv, q_pos0;
  int32_t causal, tile_q, tile_k, h;
  int64_t n_qt, n_kt;
  WindowArgs win;
};

hipError_t launch_prefill_f32(const PrefillParams& p, int head_dim, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, const PackParams& pk, int head_dim,
                               hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int head_dim, bool banded, hipStream_t stream);
hipError_t launch_kcache_band(const BandParams& p, int head_dim, hipStream_t stream);

// Size of the device array that holds the split partials of the
// allocation-free decode entry point, and its device address on the current
// device (looked up on the first call per device, then kept).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_plan(const PlanParams& p, hipStream_t stream);

}  // namespace atw
