/*
 * atw.h -- C ABI of libatw: causal attention with the per-RoPE-wavelength
 * distance window, on AMD Instinct MI355X (gfx950).
 *
 * The method (sources: "ATFlash — Per-RoPE-Wavelength Attention Windows",
 * README sections "The idea" and "Porting to something else"; "ATFlash:
 * Per-RoPE-Wavelength Attention Windows for Compute/Memory-Efficient LLM
 * Inference", arXiv abstract):
 *
 *   head dim d, h = d/2 rotation pairs, pair r = dims (r, r + d/2)
 *   (rotate-half layout); theta_r = base^(-2r/d); wavelength
 *   lambda_r = 2*pi/theta_r; window w_r = k * lambda_r.
 *   RoPE rotates pair r of the query at position n by n*theta_r and of the
 *   key at position m by m*theta_r, so its term of the score depends only on
 *   (n - m)*theta_r.  The term of pair r is kept while the query-key distance
 *   is at most w_r and is zero beyond it; the rest of the sum is kept
 *   unchanged, and the softmax over keys (running max, normalizer) is the
 *   ordinary one.  Every key stays visible through the low-frequency pairs.
 *
 *   s(n, m) = scale * sum_r [dist(n, m) <= W_r] * (q'_r k'_r + q'_{r+h} k'_{r+h})
 *   with W_r = floor(w_r), q', k' the rotated vectors, scale = 1/sqrt(d)
 *   unless given; dist = n - m (causal) or |n - m| (non-causal).
 *   O_n = sum_m softmax_m(s(n, .)) v_m over the visible keys.
 *
 * Conventions shared by every entry point:
 *   - Tensors are pre-RoPE; the rotation is applied inside the kernels as the
 *     data is loaded ("RoPE fused at load").
 *   - Element strides are given per tensor as int64 element counts; the head
 *     dimension is contiguous (stride 1).  Base pointers must be 16-byte
 *     aligned and every stride a multiple of 16 bytes / element size.
 *   - Every device pointer (workspaces included) is allocated and owned by
 *     the caller; the library allocates no device memory and keeps no state
 *     between calls except a thread-local error string.  Inputs are never written; outputs are fully
 *     written.
 *   - Calls are asynchronous on the given HIP stream (hipStream_t, passed as
 *     void*; NULL = the default stream).  Execution errors surface when the
 *     caller synchronizes.  Argument errors are detected before any launch,
 *     so an error return leaves every output untouched.
 *   - window_on = 0 is the plain causal RoPE attention path (k is ignored);
 *     k = +inf with window_on = 1 gives the same result.
 *   - Supported on the GPU: head_dim 64 or 128; dtype ATW_BF16 (bf16 in and
 *     out, fp32 accumulation, fp16 matrix-core operands) or ATW_BF16_F32OUT
 *     (the same with an fp32 output) for prefill and decode, ATW_F32 (fp32
 *     in and out, fp32 MFMA) for prefill.  Positions must be < 2^30.
 */
#ifndef ATW_H
#define ATW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATW_OK 0
#define ATW_EINVAL (-1)        /* invalid argument (null pointer, bad size, bad value) */
#define ATW_EUNSUPPORTED (-2)  /* valid but not supported (head_dim, dtype, alignment) */
#define ATW_EWORKSPACE (-3)    /* decode workspace missing or too small */
#define ATW_EHIP (-4)          /* the HIP runtime reported an error at launch */

/* element types */
#define ATW_F32 0
#define ATW_BF16 1
/* bf16 inputs with an fp32 output (o holds floats; o_strides count floats):
 * the same computation as ATW_BF16 without the final rounding of the output
 * to bf16.  Accepted by the bf16 prefill and decode entry points. */
#define ATW_BF16_F32OUT 2

/* Largest integer window; returned for every pair when the window is off or
 * k = +inf (2^62). */
#define ATW_UNBOUNDED ((int64_t)1 << 62)

/*
 * RoPE frequencies of a model whose config rescales them.  The window tables
 * are built from the RoPE base, the head dimension and the model's
 * rope_scaling ("ATFlash — Per-RoPE-Wavelength Attention Windows", README,
 * "Using the ports"); the rotation and the windows both use the rescaled
 * theta_r, so the window of pair r is w_r = k * 2*pi / theta_r.  The
 * *_rope entry points take this descriptor (host memory, read during the
 * call only) in place of rope_base; the others use ATW_ROPE_PLAIN.
 *
 *   ATW_ROPE_PLAIN   theta_r = base^(-2r/d).
 *   ATW_ROPE_LINEAR  the plain theta_r divided by factor (position
 *                    interpolation).
 *   ATW_ROPE_LLAMA3  with L = original_max_position and the plain
 *                    wavelength lambda_r = 2*pi/theta_r: pairs with
 *                    lambda_r < L / high_freq_factor keep theta_r, pairs with
 *                    lambda_r > L / low_freq_factor get theta_r / factor, and
 *                    in between theta_r' = (1 - s) theta_r / factor + s theta_r
 *                    with s = (L / lambda_r - low_freq_factor) /
 *                    (high_freq_factor - low_freq_factor) (the frequency rule
 *                    of the Llama 3.1 / 3.2 model configs).
 *   ATW_ROPE_TABLE   theta_r given per pair in theta[0 .. d/2 - 1] (any other
 *                    rescaling rule, computed by the caller).
 *
 * Every resulting theta_r must be finite, > 0 and non-increasing in r (then
 * the windows grow with r and the kept pairs at any distance are a suffix);
 * otherwise the call returns ATW_EINVAL.
 *
 * widths (optional, any kind): read only when flags has ATW_ROPE_HAS_WIDTHS
 * set; then d/2 integer windows W_r (host memory, read during the call only)
 * used in place of floor(k * 2*pi / theta_r); k_turns is then not used.  The
 * rotation still uses theta_r.  Each W_r must be >= 0 and non-decreasing in
 * r (ATW_EINVAL otherwise); values above ATW_UNBOUNDED mean unbounded.  With
 * the window off every pair is kept as usual.  This is for windows tuned or
 * stored per model rather than derived from k.
 *
 * flags: ATW_ROPE_HAS_WIDTHS or 0; any other bit set returns ATW_EINVAL.
 * (Layout note: library version 0.1 had no widths member and required this
 * word, then named reserved, to be 0; a caller built against that layout
 * therefore never has widths read past the end of its struct.)
 */
#define ATW_ROPE_PLAIN 0
#define ATW_ROPE_LINEAR 1
#define ATW_ROPE_LLAMA3 2
#define ATW_ROPE_TABLE 3
#define ATW_ROPE_HAS_WIDTHS 1   /* atw_rope.flags: the widths member is valid */

typedef struct atw_rope {
  int32_t kind;                 /* ATW_ROPE_* */
  int32_t flags;                /* ATW_ROPE_HAS_WIDTHS or 0 */
  double base;                  /* PLAIN, LINEAR, LLAMA3: > 1 */
  double factor;                /* LINEAR, LLAMA3: > 0 */
  double low_freq_factor;       /* LLAMA3: > 0 */
  double high_freq_factor;      /* LLAMA3: > low_freq_factor */
  double original_max_position; /* LLAMA3: > 0 */
  const double* theta;          /* TABLE: d/2 frequencies (host) */
  const int64_t* widths;        /* with ATW_ROPE_HAS_WIDTHS: d/2 explicit windows W_r (host) */
} atw_rope;

/* theta_r of every pair of a descriptor (d/2 values, host) -- host only. */
int atw_rope_theta(const atw_rope* rope, int32_t head_dim, double* theta_out);

/* atw_window_widths with a RoPE descriptor -- host only. */
int atw_window_widths_rope(const atw_rope* rope, int32_t head_dim, double k_turns,
                           int32_t window_on, int64_t* widths_out);

/* atw_pruned_terms with a RoPE descriptor -- host only. */
int atw_pruned_terms_rope(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim,
                          const atw_rope* rope, double k_turns, int32_t causal, int32_t window_on,
                          int64_t* pruned, int64_t* total);

/* atw_prefill with a RoPE descriptor in place of rope_base (every other
 * argument, the result and the limits as for atw_prefill). */
int atw_prefill_rope(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                     int64_t batch, int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q,
                     int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                     const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                     int32_t window_on, double softmax_scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/* atw_decode / atw_decode_banded with a RoPE descriptor in place of rope_base. */
int atw_decode_rope(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                    int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                    int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                    const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                    const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                    int32_t window_on, double softmax_scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream);
int atw_decode_banded_rope(const void* q, const void* k_bands, const void* v_cache, void* o,
                           int32_t dtype, int64_t batch, const int64_t* kv_len,
                           const int64_t* q_pos, int32_t h_q, int32_t h_kv,
                           const int32_t* kv_head_of_q, int32_t head_dim, const int64_t* q_strides,
                           const int64_t* k_strides, const int64_t* v_strides,
                           const int64_t* o_strides, const atw_rope* rope, double k_turns,
                           int32_t causal, int32_t window_on, double softmax_scale,
                           int32_t num_splits, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * atw_decode_sparse -- atw_decode_rope (k_banded = 0: row-layout K cache) or
 * atw_decode_banded_rope (k_banded = 1) composed with a block-sparse key
 * selection, as token-level selection methods make for decoding (the window
 * applies on top of them: "ATFlash: Per-RoPE-Wavelength Attention Windows
 * for Compute/Memory-Efficient LLM Inference", arXiv abstract).
 *
 *   block_mask: device uint32 [batch, h_kv, mask_words]: bit kb % 32 of word
 *     kb / 32 set = the sequence's kv head (all query heads reading it)
 *     attends keys [64 kb, 64 kb + 64).  Blocks at or beyond
 *     ceil(kv_len / 64) are ignored.  Read only, 4-byte aligned.
 *   mask_words: words per row, >= atw_block_mask_words(max kv_len).
 *
 * The split-KV partition divides each (sequence, kv head)'s selected blocks
 * evenly over num_splits; unselected keys are never read.  A query head
 * attending no key gets an output of 0.  One query token per sequence; every
 * other argument, the workspace (atw_decode_workspace_bytes), the result
 * codes and the limits as for atw_decode_rope.
 */
int atw_decode_sparse(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                      int64_t batch, const int64_t* kv_len, const int64_t* q_pos, int32_t h_q,
                      int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                      const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                      const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                      int32_t window_on, double softmax_scale, int32_t num_splits,
                      const uint32_t* block_mask, int64_t mask_words, int32_t k_banded,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * atw_prefill -- windowed causal (or non-causal) attention for a block of
 * queries against a key/value sequence ("The idea": the window is a slice of
 * the query-key contraction axis; "Porting to something else": the pair loop
 * starts at the window boundary and the rotation is fused at load).
 *
 *   q  [batch, h_q,  n_q,  head_dim]   query i is at position q_pos0 + i
 *   k  [batch, h_kv, n_kv, head_dim]   key j is at position j
 *   v  [batch, h_kv, n_kv, head_dim]
 *   o  [batch, h_q,  n_q,  head_dim]   written
 *   *_strides[3] = element strides of (batch, head, token).
 *   kv_head_of_q: host array [h_q] giving the kv head each query head reads
 *     (grouped-query attention); NULL = h // (h_q / h_kv).
 *   causal: 1 = key j visible iff j <= query position (a chunked prefill
 *     passes q_pos0 = tokens already cached and n_kv = q_pos0 + n_q);
 *     0 = every key visible, window on |n - m|.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   workspace: device buffer of at least atw_prefill_workspace_bytes(...)
 *     bytes (ATW_BF16: the keys rotated once and the values, both re-ordered
 *     into matrix-core operand order, 64-key tiles, as fp16 scaled by a power
 *     of two per (batch, kv head) when |k| or |v| reaches 2^14, plus the
 *     per-chunk maxima that choose those scales; ATW_F32: none needed, may
 *     be NULL).  Contents on entry are ignored; overwritten by the call.
 *   ATW_BF16 arithmetic: matrix-core operands fp16 (rotated queries and keys,
 *     values, softmax weights), accumulation fp32, output bf16
 *     (ATW_BF16_F32OUT: fp32).
 * Requires n_q >= 0, n_kv >= 1, q_pos0 >= 0, h_q % h_kv == 0 without a map,
 * rope_base > 1, k_turns > 0 when window_on, batch <= 65535.  n_q = 0
 * launches nothing.
 */
int atw_prefill(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                int64_t batch, int64_t n_q, int64_t n_kv, int64_t q_pos0,
                int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                const int64_t* o_strides,
                double rope_base, double k_turns, int32_t causal, int32_t window_on,
                double softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * atw_prefill_sparse -- atw_prefill composed with a block-sparse key
 * selection: a token-level selection (as made by dynamic-sparse methods) is
 * orthogonal to the frequency-level window, which therefore applies on top
 * of it ("ATFlash: Per-RoPE-Wavelength Attention Windows for
 * Compute/Memory-Efficient LLM Inference", arXiv abstract).
 *
 * Blocks are ATW_SPARSE_BLOCK = 64 query rows by 64 keys, counted from the
 * start of the call's tensors (query block qb = rows [64 qb, 64 qb + 64) of
 * q, key block kb = keys [64 kb, 64 kb + 64) of k).  A query attends key m
 * iff the block of m is selected for the query's block, and (causal) m is
 * not after the query's position; inside that set the per-pair window
 * applies as in atw_prefill, and keys outside it are out of the softmax.  A
 * query row that attends no key gets an output of 0.
 *
 *   block_mask: device uint32 [batch, h_q, ceil(n_q / 64), W] with
 *     W = atw_block_mask_words(n_kv); bit kb % 32 of word kb / 32 of row
 *     (b, hq, qb) set = query block qb of query head hq attends key block kb.
 *     Bits for key blocks at or beyond ceil(n_kv / 64) are ignored.  Read
 *     only, owned by the caller, 4-byte aligned.
 *
 * Every other argument, the workspace, the result codes and the limits as
 * for atw_prefill_rope; dtype ATW_BF16 only (ATW_EUNSUPPORTED otherwise).
 * With every bit of the mask set the output is bit-identical to atw_prefill.
 */
#define ATW_SPARSE_BLOCK 64
int atw_prefill_sparse(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                       int64_t batch, int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t h_q,
                       int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                       const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                       const int64_t* o_strides, const atw_rope* rope, double k_turns, int32_t causal,
                       int32_t window_on, double softmax_scale, const uint32_t* block_mask,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Words per block_mask row: ceil(ceil(n_kv / 64) / 32); 0 for n_kv <= 0. */
int64_t atw_block_mask_words(int64_t n_kv);

/*
 * atw_pruned_terms_sparse -- host only.  atw_pruned_terms_rope over the cells
 * a block-sparse selection attends, for one (batch, query head):
 * block_mask is host uint32 [ceil(n_q / 64), atw_block_mask_words(n_kv)]
 * (one head's rows of atw_prefill_sparse's mask).  Writes the pruned and
 * total pair-terms of the attended cells (closed form per selected block
 * and pair).
 */
int atw_pruned_terms_sparse(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim,
                            const atw_rope* rope, double k_turns, int32_t causal, int32_t window_on,
                            const uint32_t* block_mask, int64_t* pruned, int64_t* total);

/* Workspace bytes atw_prefill needs: ATW_BF16: 2 * batch * h_kv *
 * ceil(n_kv / 64) * 64 * head_dim * 2 (one copy of K and V) + batch * h_kv *
 * 256 (range maxima); ATW_F32: 0. */
size_t atw_prefill_workspace_bytes(int32_t dtype, int64_t batch, int32_t h_kv, int64_t n_kv,
                                   int32_t head_dim);

/*
 * atw_decode -- one query token per sequence against a pre-RoPE KV cache,
 * split over the key axis (split-KV) and merged by a combine pass.  The
 * window acts in the key loads: for each key only the pair slice inside the
 * window at that key's distance is read ("The idea": the out-of-window prefix
 * of a key is never loaded).
 *
 *   q       [batch, h_q, head_dim]           strides q_strides[2] (batch, head)
 *   k_cache [batch, h_kv, L, head_dim]       strides k_strides[3] (batch, head, token)
 *   v_cache [batch, h_kv, L, head_dim]       strides v_strides[3]
 *   o       [batch, h_q, head_dim]           strides o_strides[2], written
 *   kv_len  host int64 [batch]: keys 0..kv_len[b]-1 of sequence b are valid (>= 1)
 *   q_pos   host int64 [batch]: position of sequence b's query; causal
 *           requires q_pos[b] >= kv_len[b] - 1 (all cached keys visible).
 *   num_splits: key-axis splits per (sequence, kv head), 1..1024; the
 *           splits cover consecutive key ranges of about kv_len/num_splits
 *           keys (boundaries at multiples of 4 keys).
 *   workspace: device buffer of at least atw_decode_workspace_bytes(...)
 *           bytes for the per-split partial results (max, sum, unnormalised
 *           output); contents on entry are ignored.
 * batch <= 256; at most 16 query heads per kv head.  dtype ATW_BF16 or
 * ATW_BF16_F32OUT.
 */
int atw_decode(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
               int64_t batch, const int64_t* kv_len, const int64_t* q_pos,
               int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
               const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
               const int64_t* o_strides,
               double rope_base, double k_turns, int32_t causal, int32_t window_on,
               double softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
               void* stream);

/* Workspace bytes atw_decode needs: batch * h_q * num_splits * (head_dim + 4) * 4. */
size_t atw_decode_workspace_bytes(int64_t batch, int32_t h_q, int32_t head_dim, int32_t num_splits);

/*
 * atw_decode_noalloc -- atw_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, result and kernels, without the
 * workspace.  The per-split partials go to a device array the library holds
 * on each GPU it runs on until the process ends (atw_decode_noalloc_max_bytes()
 * = 16 MiB); its address is looked up on the first call on each device.  The
 * call allocates nothing.
 *   Returns ATW_EWORKSPACE, before any launch, when the partials
 *   (atw_decode_workspace_bytes(batch, h_q, head_dim, num_splits)) exceed the
 *   array.  Every call on one GPU uses that GPU's one array: calls that overlap
 *   in time on one GPU (other streams, other threads) race and must not be
 *   issued; calls in one stream are ordered and safe.  Each call writes every
 *   partial it reads, so nothing carries over from an earlier call.
 */
int atw_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                       int64_t batch, const int64_t* kv_len, const int64_t* q_pos,
                       int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                       const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                       const int64_t* o_strides,
                       double rope_base, double k_turns, int32_t causal, int32_t window_on,
                       double softmax_scale, int32_t num_splits, void* stream);

/* Bytes of atw_decode_noalloc's per-device array (the largest partials it takes). */
size_t atw_decode_noalloc_max_bytes(void);

/*
 * atw_decode_banded -- atw_decode over a pair-banded K cache.  The memory
 * system of this GPU moves whole 128-byte lines; in the row layout every line
 * of a key row holds dims of all pairs, so skipping the out-of-window pairs
 * of a key ("The idea": the out-of-window prefix is never loaded) saves no
 * memory traffic.  In the banded layout band c (c = 0 .. head_dim/16 - 1)
 * holds, per key, dims [8c, 8c+8) followed by dims [h+8c, h+8c+8) (h =
 * head_dim/2), i.e. rotation pairs 8c .. 8c+7, 32 bytes per key, keys
 * contiguous:
 *
 *   k_bands [batch, h_kv, head_dim/16, L, 16]   k_strides[3] = element strides
 *            of (batch, head, band); the token stride is 16 elements.
 *
 * A line then holds one band of 4 consecutive keys and is fetched only when
 * the band is inside the window for one of them.  The splits are sized for
 * equal bytes rather than equal keys (a split far from the query needs fewer
 * bands per key and covers more keys).  Every other argument, the result and
 * the limits are those of atw_decode (same output up to fp32 rounding of the
 * split merge; bit-identical when the window is off).
 */
int atw_decode_banded(const void* q, const void* k_bands, const void* v_cache, void* o,
                      int32_t dtype, int64_t batch, const int64_t* kv_len, const int64_t* q_pos,
                      int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                      const int64_t* q_strides, const int64_t* k_strides,
                      const int64_t* v_strides, const int64_t* o_strides, double rope_base,
                      double k_turns, int32_t causal, int32_t window_on, double softmax_scale,
                      int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * atw_decode_multi -- decode of q_len query tokens per sequence at
 * consecutive positions q_pos[b], q_pos[b] + 1, ..., q_pos[b] + q_len - 1
 * (the draft tokens that multi-token prediction or speculative decoding
 * verifies in one step; "MiMo-V2.6-Pro-RL and MTP": the windows are used
 * with MTP drafts), causal: token j of sequence b sees keys 0 ..
 * q_pos[b] + j of its cache (the drafts' own keys appended before the call),
 * with the window measured from its own position.  Token j's output equals
 * that of atw_decode with q_pos = q_pos[b] + j and kv_len = q_pos[b] + j + 1.
 *
 *   q [batch, q_len, h_q, d]    q_strides[3] = element strides of (batch, head,
 *                               token) (the token stride a multiple of 16 bytes)
 *   o [batch, q_len, h_q, d]    o_strides[3] likewise
 *   k_cache: row layout [batch, h_kv, L, d] (k_banded = 0) or the pair-banded
 *   layout of atw_decode_banded (k_banded = 1); v_cache as for atw_decode;
 *   kv_len[b] >= 1 with q_pos[b] + q_len - 1 >= kv_len[b] - 1.
 *   workspace: atw_decode_multi_workspace_bytes(...) bytes.
 *
 * q_len 1..16; the (query head, token) pairs of one kv head form the columns of
 * the score MFMA, so tokens are processed in groups of 16 / (query heads per
 * kv head), one kernel pass over the caches per group.  RoPE frequencies from
 * the descriptor (see atw_rope).  Other limits as for atw_decode.
 */
size_t atw_decode_multi_workspace_bytes(int64_t batch, int32_t q_len, int32_t h_q, int32_t head_dim,
                                        int32_t num_splits);
int atw_decode_multi(const void* q, const void* k_cache, const void* v_cache, void* o, int32_t dtype,
                     int64_t batch, int32_t q_len, const int64_t* kv_len, const int64_t* q_pos,
                     int32_t h_q, int32_t h_kv, const int32_t* kv_head_of_q, int32_t head_dim,
                     const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                     const int64_t* o_strides, int32_t k_banded, const atw_rope* rope,
                     double k_turns, int32_t window_on, double softmax_scale, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * atw_kcache_band -- copy keys [t0, t0 + n_tokens) of a row-layout K cache
 * (k_rows [batch, h_kv, L, head_dim], row_strides = (batch, head, token)) into
 * a pair-banded one (k_bands as for atw_decode_banded, band_strides =
 * (batch, head, band)).  Use it to band a whole cache or to append the keys
 * of each new step.  The two buffers must not overlap.  dtype ATW_BF16,
 * head_dim 64 or 128, t0 + n_tokens <= 2^30; n_tokens = 0 launches nothing.
 * Asynchronous on stream.
 */
int atw_kcache_band(const void* k_rows, void* k_bands, int32_t dtype, int64_t batch, int32_t h_kv,
                    int32_t head_dim, int64_t t0, int64_t n_tokens, const int64_t* row_strides,
                    const int64_t* band_strides, void* stream);

/*
 * atw_pruned_terms -- host only.  Number of pruned and total pair-terms
 * (one term = one (query, key, pair) triple) per (batch, query head) over the
 * visible cells of a prefill call with the same arguments (decode: n_q = 1,
 * q_pos0 = q_pos, n_kv = kv_len).  Exact closed form (one arithmetic series
 * per pair), input independent ("The idea": the cost is known before
 * running).  Writes *pruned and *total.
 */
int atw_pruned_terms(int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t head_dim,
                     double rope_base, double k_turns, int32_t causal, int32_t window_on,
                     int64_t* pruned, int64_t* total);

/*
 * atw_window_widths -- host only.  Integer windows W_r = floor(k * 2*pi /
 * theta_r), r = 0..head_dim/2-1, computed in IEEE double and written to
 * widths_out (host int64 [head_dim/2]); ATW_UNBOUNDED when the window is off
 * or k = +inf.  Any even head_dim in 2..256 is accepted.
 */
int atw_window_widths(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                      int64_t* widths_out);

/*
 * atw_window_plan -- host only.  Tile plan ("Porting to something else": the
 * retained prefix per key tile): for query tile a (rows a*tile_q ...) and key
 * tile b (keys b*tile_k ...) writes plan_out[(a*n_kt + b)*2 + {0,1}] =
 * (r_any, r_full): pairs below r_any are pruned for every visible cell of the
 * tile, pairs from r_full on are kept for every visible cell; (-1, -1) for a
 * tile without a visible cell.  n_qt = ceil(n_q/tile_q), n_kt =
 * ceil(n_kv/tile_k); plan_out is host int32 [n_qt * n_kt * 2].
 */
int atw_window_plan(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                    int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t causal,
                    int32_t tile_q, int32_t tile_k, int32_t* plan_out);

/*
 * atw_window_plan_device -- the same tile plan, computed on the GPU by the
 * device code the prefill kernels use for their per-tile pair ranges and
 * per-cell pair masks.  plan_out: device int32 [n_qt * n_kt * 2] as above;
 * pruned_out: device int64 [n_qt * n_kt], the number of pruned pair-terms of
 * each tile as the kernels' masks count them (sums to atw_pruned_terms).
 * n_q * n_kv must be <= 2^40.  Asynchronous on stream.
 */
int atw_window_plan_device(int32_t head_dim, double rope_base, double k_turns, int32_t window_on,
                           int64_t n_q, int64_t n_kv, int64_t q_pos0, int32_t causal,
                           int32_t tile_q, int32_t tile_k, int32_t* plan_out, int64_t* pruned_out,
                           void* stream);

/* Message of the last error on the calling thread ("" if none). */
const char* atw_last_error(void);

/* Library version string ("atw 0.3 (gfx950)": atw_rope carries the optional
 * widths pointer since 0.2, read only under ATW_ROPE_HAS_WIDTHS since 0.3;
 * bf16 prefill and decode use fp16 matrix-core operands since 0.3). */
const char* atw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATW_H */
