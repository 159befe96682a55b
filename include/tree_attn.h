/*
 * tree_attn.h -- C ABI of libtreeattn.so: tree-masked decode attention for
 * AMD MI355X (gfx950).
 *
 * One pass of the tree-verify step of speculative decoding: every draft-tree
 * node (query) attends the KV cache under an explicit per-node mask, with
 * GQA, an online softmax over split KV ranges, and a log-sum-exp merge of
 * the split results.  A second entry point does the same over an
 * affine-quantized (4/8-bit) KV cache with optional attention sinks.
 *
 * Sources, cited by page title and section:
 *   [TA]  "tree_attention.metal" (mlx-native 0.9.1): header comment,
 *         TreeAttentionParams, tree_attention_impl.
 *   [OPS] "ops/tree_attention.rs" (mlx-native 0.9.2): module doc, mask
 *         constants, TreeAttentionParams, validate_buffers, validate_params,
 *         tree_attention() doc, tmp_buffer_bytes.
 *   [FQS] "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0): module doc
 *         (Layout, Mask variants, dispatch invariants), base and float-mask
 *         kernel macros.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked DEVICE are device memory owned by the caller (for
 *   example torch tensors); HOST pointers are host memory.  The library
 *   allocates nothing, keeps no pointer after returning, and never
 *   synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the
 *   null stream) and is complete when that stream reaches it.
 * - Every `*_bytes` argument is the size of the caller's buffer.  It is
 *   compared with the size the call needs, computed in 64-bit arithmetic
 *   with overflow checks ([OPS] validate_buffers uses checked multiplies for
 *   the same reason).
 * - All arguments are validated on the host before anything is enqueued.
 *   On any error the function returns a negative TA_* code, enqueues
 *   nothing, and tree_attn_last_error() describes the problem.
 * - Device pointers must be 16-byte aligned (torch allocations are).
 * - Calls on one stream are ordered; calls sharing an output or partial
 *   buffer on different streams race and are the caller's to order.
 * - Thread-safe: the library state is the per-thread error string and, for
 *   tree_attn_forward_noalloc only, the device address of its static
 *   scratch on each device (looked up once).
 * - Only tree_attn_forward_noalloc uses memory the caller did not pass: a
 *   static device buffer that every device the library runs on holds until
 *   the process ends.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the library; everything else in it is hidden. */
#define TA_API __attribute__((visibility("default")))

/* Return codes. */
#define TA_OK 0
#define TA_EINVAL (-1)       /* an argument is invalid (shape, pointer, topology) */
#define TA_ESIZE (-2)        /* a buffer is smaller than the call needs */
#define TA_EOVERFLOW (-3)    /* a size computation overflows 64 bits */
#define TA_EUNSUPPORTED (-4) /* valid but not implemented (head_dim, dtype, ...) */
#define TA_EHIP (-5)         /* the HIP runtime reported an error on launch */

/* Element types. */
#define TA_F32 0
#define TA_F16 1
#define TA_BF16 2 /* bfloat16: quantized path element type, merge output */

/* Mask sentinels ([OPS] mask constants).  A mask cell <= TA_MASKED excludes
 * the key; any larger value is ADDED to the scaled logit (0 = attended). */
#define TA_MASKED (-65504.0f)
#define TA_ATTENDED 0.0f

/* Mask kinds of tree_attn_quant_forward_ex. */
#define TA_MASK_NONE 0 /* no mask buffer: the implicit causal rule */
#define TA_MASK_F16 1  /* additive bias in the element type T ([FQS] float-mask
                          macro); fp16 when T is fp16 */
#define TA_MASK_BOOL 2 /* u32 visibility words ([FQS] bool-mask macro) */

/*
 * Bytes of the split-KV partial-result scratch for `nwg` splits:
 *   n_heads * q_l * nwg * (head_dim + 2) * 4, saturating at SIZE_MAX.
 * This is the size formula of [OPS] tmp_buffer_bytes with the split count
 * as an argument.  For the quantized path pass n_heads = batch * n_q_heads.
 * Layout (this library's own): float O[nwg][nrows][head_dim] holding the
 * unnormalised output of each split, then float SM[nwg][nrows][2] holding
 * (S, M): the split's softmax denominator and its running maximum in base-2
 * units (log2(e) * max logit; -inf for a split that saw no key).
 * nrows = n_heads * q_l and row r is the output row (r = i * n_heads + h on
 * the fp path, r = q_idx * q_l + i on the quantized path).
 */
TA_API size_t tree_attn_partials_bytes(uint32_t n_heads, uint32_t head_dim,
                                uint32_t q_l, uint32_t nwg);

/*
 * Optional tail of the partials buffer.  When tree_attn_forward gets an
 * explicit mask, nwg > 1 and a partials buffer of at least
 * tree_attn_partials_bytes(...) + TA_RANGE_BYTES bytes, it may first scan
 * the mask for its first and last live key (one extra small kernel, results
 * in those TA_RANGE_BYTES) and split only the tiles between them: a mask
 * whose dead cells form a prefix or suffix of every row (a sliding window
 * written as a mask) then costs neither K/V fetches nor idle splits ("tree_attention.metal",
 * tree_attention_impl: a chunk whose cells are all masked is skipped).  It
 * does so when the K/V bytes read are at least 64 MiB and at least 32 times
 * the mask bytes; otherwise, or without the tail, every tile is split and
 * fetched and a fully masked tile only skips its arithmetic.  The result
 * meets the same contract either way; the tail's contents after the call
 * are unspecified.
 */
#define TA_RANGE_BYTES 2048

/*
 * A split count for tree_attn_forward that fills `num_cus` compute units
 * (0 means 256, MI355X), given the problem shape.  Pure function of its
 * arguments (no device query).  Always >= 1.  Callers pass the result as
 * `nwg` to the forward call, size the partials with it and pass it to
 * tree_attn_reduce.
 */
TA_API uint32_t tree_attn_pick_nwg(uint32_t n_heads, uint32_t n_kv_heads,
                            uint32_t head_dim, uint32_t kv_seq_len,
                            uint32_t q_l, int kv_dtype, uint32_t num_cus);

/* The same for tree_attn_quant_forward (4-bit codes with an fp16 mask
 * assumed for the residency of a workgroup). */
TA_API uint32_t tree_attn_quant_pick_nwg(uint32_t batch, uint32_t n_q_heads,
                                  uint32_t n_kv_heads, uint32_t dim,
                                  uint32_t kv_seq_len, uint32_t q_l,
                                  uint32_t num_cus);

/*
 * The split count for tree_attn_quant_forward(_ex) with the kernel variant
 * the call will run: bits, group_size and mask_kind (TA_MASK_*) set its
 * registers and LDS, and so how many workgroups a CU holds at once.  That
 * number comes from the HIP runtime's occupancy query for the variant on the
 * current device (capped at two wavefronts per SIMD); without a device it is
 * estimated from the variant's LDS size.  With a sliding window pass min(window_size, kv_seq_len) as
 * kv_seq_len.  Always >= 1.
 */
TA_API uint32_t tree_attn_quant_pick_nwg_ex(uint32_t batch, uint32_t n_q_heads,
                                     uint32_t n_kv_heads, uint32_t dim,
                                     uint32_t kv_seq_len, uint32_t q_l, uint32_t bits,
                                     uint32_t group_size, int mask_kind, int q_dtype,
                                     uint32_t num_cus);

/*
 * Tree-attention forward pass ([TA] tree_attention_impl; [OPS]
 * tree_attention()).  For every node i < q_l and query head h < n_heads,
 * with kv head hk = h / (n_heads / n_kv_heads) ([TA] GQA mapping):
 *   logit_j = scale * dot(q[h, i, :], k[hk, j, :]) + mask[i, j]  for j < kv_seq_len
 *   out[i, h, :] = sum_j softmax(logit)_j * v[hk, j, :]
 * where keys with mask[i, j] <= TA_MASKED are left out, and a row that
 * keeps no key yields zeros ([TA] writes 0 when the sum S is 0).
 *
 *   q     DEVICE f32  [n_heads, q_l, head_dim]               (q_bytes)
 *   k, v  DEVICE kv_dtype (TA_F32 or TA_F16)
 *                     [n_kv_heads, kv_capacity, head_dim]    (kv_bytes each)
 *         Rows j >= kv_seq_len are never read.
 *   mask  DEVICE f32  [q_l, mask_stride], row-major, mask_stride >= kv_seq_len
 *         (mask_bytes >= q_l * mask_stride * 4); cells j >= kv_seq_len are
 *         never read ([OPS] tree_attention() doc).  mask == NULL selects the
 *         implicit causal rule of [TA] header: node i sees key j iff
 *         j <= kv_seq_len - q_l + i.  An explicit mask that encodes that
 *         same rule gives a byte-identical result.
 *   nwg   number of KV splits (>= 1).  nwg == 1: the final result is written
 *         to `out` and `partials` may be NULL.  nwg > 1: the per-split
 *         results go to `partials` (size tree_attn_partials_bytes(n_heads,
 *         head_dim, q_l, nwg)), `out` is not touched and may be NULL, and
 *         tree_attn_reduce must follow on the same stream.
 *   out   DEVICE f32  [q_l, n_heads, head_dim] -- query-outer, head-inner,
 *         NOT Q's layout ([OPS] tree_attention() doc).
 *
 * head_dim must be 128, 256 or 512 ([OPS] validate_params); n_heads and
 * n_kv_heads > 0 with n_heads % n_kv_heads == 0; kv_seq_len > 0;
 * kv_capacity >= kv_seq_len; q_l > 0.  fp16 K/V are contracted with fp16
 * operands and fp32 accumulation (Q rounded to fp16 after scaling); fp32 K/V
 * are contracted in fp32.
 */
TA_API int tree_attn_forward(const float *q, size_t q_bytes, const void *k,
                      const void *v, int kv_dtype, size_t kv_bytes,
                      const float *mask, size_t mask_bytes, float *partials,
                      size_t partials_bytes, float *out, size_t out_bytes,
                      uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                      uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
                      uint32_t mask_stride, float scale, uint32_t nwg,
                      void *stream);

/*
 * Causal (sliding-window) decode without a mask buffer: the implicit rule
 * of [TA] header, which flash_attn_vec computes from abs_pos = kv_seq_len -
 * q_l + i.  Node i (query position abs_pos) sees key j iff
 *   window_start <= j <= abs_pos,
 * with one window_start for every row (the header's byte-identity contract
 * pairs it with an explicit mask that is 0.0f on [window_start, abs_pos]).
 * A node whose abs_pos < window_start sees nothing and yields zeros.
 * Arguments and results as tree_attn_forward with mask == NULL, plus:
 *
 *   window_start  first key any row may see; 0 gives the plain causal rule
 *                 (the same call as tree_attn_forward with mask == NULL).
 *                 Must be < kv_seq_len (TA_EINVAL otherwise).  Keys below
 *                 the 32-key (16 at head_dim 512 with fp32 K/V) tile that
 *                 holds window_start are not read, and a split count from
 *                 tree_attn_pick_nwg(..., kv_seq_len - window_start, ...)
 *                 sizes the splits to the window.  The result equals
 *                 tree_attn_forward with the explicit window mask to
 *                 rounding, and bit for bit when window_start lies in the
 *                 first tile (both calls then split the same keys).
 */
TA_API int tree_attn_decode(const float *q, size_t q_bytes, const void *k,
                     const void *v, int kv_dtype, size_t kv_bytes, float *partials,
                     size_t partials_bytes, float *out, size_t out_bytes,
                     uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                     uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
                     uint32_t window_start, float scale, uint32_t nwg, void *stream);

/*
 * Log-sum-exp merge of split partial results (the reduce pass that [TA]
 * header and [OPS] tree_attention() run after the main kernel).  For each
 * row r, over the splits w with S_w > 0:
 *   M* = max_w M_w,  S* = sum_w S_w 2^(M_w - M*),
 *   out[r, :] = sum_w O_w[r, :] 2^(M_w - M*) / S*,  and 0 if no split saw a key.
 *
 *   partials  DEVICE f32, layout of tree_attn_partials_bytes, for `nrows`
 *             rows, `head_dim` columns and `nwg` splits.
 *   out       DEVICE out_dtype (TA_F32, TA_F16 or TA_BF16) [nrows, head_dim];
 *             fp16 and bf16 results are rounded to nearest even.
 * head_dim must be a multiple of 4 in [4, 512]; nwg >= 1.
 */
TA_API int tree_attn_reduce(const float *partials, size_t partials_bytes, void *out,
                     int out_dtype, size_t out_bytes, uint32_t nrows,
                     uint32_t head_dim, uint32_t nwg, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * tree_attn_forward followed by tree_attn_reduce (out_dtype TA_F32) in one
 * call, with the split partials kept in a static device buffer of
 * TA_NOALLOC_SCRATCH_BYTES that the library owns instead of a caller
 * buffer.  Arguments, layouts and rules are tree_attn_forward's, without
 * partials/partials_bytes; `out` ([q_l, n_heads, head_dim] f32) is always
 * written, for every nwg.  Results are identical, bit for bit, to
 * tree_attn_forward + tree_attn_reduce with the same nwg.
 *
 * - nwg must satisfy tree_attn_partials_bytes(n_heads, head_dim, q_l, nwg)
 *   <= TA_NOALLOC_SCRATCH_BYTES, else TA_ESIZE (nothing enqueued).  nwg == 1
 *   uses no scratch.
 * - No call allocates or frees memory.  The first call on a device looks up
 *   the buffer's device address there (hipGetSymbolAddress; the stream's
 *   device, the current device for the null stream) and keeps it; a failed
 *   lookup returns TA_EHIP.
 * - One buffer per GPU, shared by every call on that GPU: calls that can
 *   overlap on one GPU (different streams, or host threads not ordered by
 *   one stream) race and give wrong results.  Calls on one stream are safe.
 *   The buffer keeps the last call's contents; nothing in it needs to start
 *   at zero (every split writes all of its partial rows before the merge
 *   reads them).
 */
#define TA_NOALLOC_SCRATCH_BYTES (64ull << 20)
TA_API int tree_attn_forward_noalloc(const float *q, size_t q_bytes, const void *k,
                              const void *v, int kv_dtype, size_t kv_bytes,
                              const float *mask, size_t mask_bytes, float *out,
                              size_t out_bytes, uint32_t n_heads, uint32_t n_kv_heads,
                              uint32_t head_dim, uint32_t kv_seq_len,
                              uint32_t kv_capacity, uint32_t q_l, uint32_t mask_stride,
                              float scale, uint32_t nwg, void *stream);

/*
 * Attention over an affine-quantized K/V cache ([FQS] Layout, base and
 * float-mask kernel macros), generalised to q_l queries per head and split
 * over KV ranges like tree_attn_forward.  For query row q_idx = b*n_q_heads
 * + h (b < batch) and node i < q_l, kv stream kv = q_idx / (n_q_heads /
 * n_kv_heads) ([FQS] GQA mapping), element d of token t is
 *   x = scale_g * code + bias_g,  g = d / group_size,
 *   code = (word[d / pf] >> ((d % pf) * bits)) & (2^bits - 1),  pf = 32/bits,
 * and
 *   logit_t = scale * dot(q[q_idx, i, :], K_t) + maskv(q_idx, i, t)
 *   out[q_idx, i, :] = softmax over {keys, sink} of the values (sink value 0)
 * The sink, when `sinks` is given, is one virtual key with raw logit
 * sinks[q_idx % n_q_heads] (no scale, no mask) ([FQS] accumulator start).
 * T, the element type of q, the scales, biases, mask and out ([FQS] kernels
 * are generic in it), is fp16, bf16 or fp32 (q_dtype).
 * maskv is an additive bias in T ([FQS] float-mask macro): cell at element
 * offset q_idx*mask_head_stride + i*mask_stride + t; cells <= TA_MASKED
 * exclude the key.  mask_head_stride = q_l*mask_stride gives a per-row
 * mask ([FQS] shape [B*nQ, tokens] when q_l = 1); 0 broadcasts one
 * [q_l, mask_stride] tree mask to every head.  mask == NULL selects the
 * implicit causal rule (every token when q_l = 1).
 *
 *   q          DEVICE T   [batch*n_q_heads, q_l, dim]                (q_bytes)
 *   k_packed   DEVICE u32 [batch*n_kv_heads, kv_capacity, dim/pf]    (kv_bytes[0])
 *   k_scales   DEVICE T   [batch*n_kv_heads, kv_capacity, dim/group] (kv_bytes[1])
 *   k_biases   DEVICE T   same shape as k_scales                     (kv_bytes[2])
 *   v_packed, v_scales, v_biases: same shapes                (kv_bytes[3..5])
 *   sinks      DEVICE f32 [n_q_heads] or NULL                        (sinks_bytes)
 *   mask       DEVICE T or NULL, aligned to sizeof(T)                (mask_bytes)
 *   partials   as tree_attn_forward with n_heads = batch*n_q_heads
 *   out        DEVICE T   [batch*n_q_heads, q_l, dim], written iff nwg == 1
 *
 * q_dtype is TA_F16, TA_BF16 or TA_F32 (T).  Q enters the matrix
 * instructions as fp16: exactly for fp16, converted for bf16 (exact for
 * magnitudes in fp16's normal range), as an fp16 hi + lo pair for fp32.
 * Scales, biases and the mask are used in fp32; out is rounded to nearest
 * even.  bits is 4 or 8; dim is 64, 96, 128, 256 or 512 ([FQS]
 * instantiations); group_size is 32, 64 or 128 and divides dim (so 32 at
 * dim 96); kv_capacity >= kv_seq_len > 0 (and even when dim/group_size is
 * odd with a 2-byte T: group_size == dim, or dim 96); mask_stride >= kv_seq_len when a mask is given.  With
 * nwg > 1 follow with tree_attn_reduce(out_dtype = q_dtype, nrows =
 * batch*n_q_heads*q_l, head_dim = dim).
 */
TA_API int tree_attn_quant_forward(
    const void *q, int q_dtype, size_t q_bytes, const uint32_t *k_packed,
    const void *k_scales, const void *k_biases, const uint32_t *v_packed,
    const void *v_scales, const void *v_biases, const size_t kv_bytes[6],
    const float *sinks, size_t sinks_bytes, const void *mask,
    size_t mask_bytes, uint64_t mask_head_stride, uint32_t mask_stride,
    float *partials, size_t partials_bytes, void *out, size_t out_bytes,
    uint32_t batch, uint32_t n_q_heads, uint32_t n_kv_heads, uint32_t dim,
    uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l, uint32_t bits,
    uint32_t group_size, float scale, uint32_t nwg, void *stream);

/*
 * tree_attn_quant_forward with the other mask kind and the sliding window of
 * [FQS] (bool-mask macro; the causal / sliding-window gate of the base,
 * bool- and float-mask macros).  Arguments as tree_attn_quant_forward, plus:
 *
 *   mask_kind    TA_MASK_NONE (mask must be NULL), TA_MASK_F16 (mask is the
 *                fp16 additive bias described above) or TA_MASK_BOOL (mask
 *                is DEVICE u32, same cell layout: a zero word drops token t
 *                for that row, any other value keeps it with no bias).
 *                The buffer must hold the last cell, (batch*n_q_heads - 1)
 *                * mask_head_stride + (q_l - 1) * mask_stride + kv_seq_len
 *                - 1, in elements of 2 (F16) or 4 (BOOL) bytes, and be
 *                aligned to its element size.
 *   window_size  0 keeps every token; W > 0 keeps token t only if
 *                t + W > kv_seq_len - 1 (the last W tokens), for every row,
 *                on top of the mask.  W >= kv_seq_len keeps every token.
 *                Tokens before the window are not read at all, and a split
 *                count from tree_attn_quant_pick_nwg(..., min(W, kv_seq_len),
 *                ...) sizes the splits to the window.
 *
 * Errors as tree_attn_quant_forward, and TA_EINVAL for an unknown mask_kind
 * or a mask pointer that does not match it (NULL iff TA_MASK_NONE).
 * tree_attn_quant_forward(...) is this call with mask_kind = mask ?
 * TA_MASK_F16 : TA_MASK_NONE and window_size = 0.
 */
TA_API int tree_attn_quant_forward_ex(
    const void *q, int q_dtype, size_t q_bytes, const uint32_t *k_packed,
    const void *k_scales, const void *k_biases, const uint32_t *v_packed,
    const void *v_scales, const void *v_biases, const size_t kv_bytes[6],
    const float *sinks, size_t sinks_bytes, const void *mask, int mask_kind,
    size_t mask_bytes, uint64_t mask_head_stride, uint32_t mask_stride,
    uint32_t window_size, float *partials, size_t partials_bytes, void *out,
    size_t out_bytes, uint32_t batch, uint32_t n_q_heads, uint32_t n_kv_heads,
    uint32_t dim, uint32_t kv_seq_len, uint32_t kv_capacity, uint32_t q_l,
    uint32_t bits, uint32_t group_size, float scale, uint32_t nwg, void *stream);

/*
 * Build the explicit tree mask on the device ([TA] header: chains, fixed
 * and dynamic trees all reduce to a [q_l, kv_seq_len] mask of 0 / -65504).
 * Node i sits at KV position kv_seq_len - q_l + i; row i is TA_ATTENDED on
 * the prefix [0, kv_seq_len - q_l), on the positions of node i's ancestors
 * and on its own position, and TA_MASKED everywhere else, including the
 * padding columns [kv_seq_len, mask_stride).
 *
 *   parents  HOST i32 [q_l]: parents[0] == -1 and 0 <= parents[i] < i.
 *            Read before the call returns; not retained.
 *   mask     DEVICE f32 [q_l, mask_stride]   (mask_bytes >= q_l*mask_stride*4)
 * 1 <= q_l <= 1024 (else TA_EUNSUPPORTED), q_l <= kv_seq_len <= mask_stride.
 */
TA_API int build_tree_mask(const int32_t *parents, uint32_t q_l, uint32_t kv_seq_len,
                    uint32_t mask_stride, float *mask, size_t mask_bytes,
                    void *stream);

/* Message for the last error returned on the calling thread ("" if none). */
TA_API const char *tree_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
