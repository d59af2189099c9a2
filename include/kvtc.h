/*
 * kvtc.h -- transform-coded low-bit KV cache and decode attention over it,
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes (the pages it follows):
 *   - encode: each key/value x (head_dim = 128) of KV head h is projected onto
 *     the head's basis P_h (d x r, orthonormal columns, random-sign Hadamard
 *     already folded in): c = P_h^T x; the r coordinates are quantized with the
 *     head's b-bit uniform quantizer (per-token fp16 min and step) and
 *     bit-packed at a fixed per-token width.
 *     [KV-COBRA project page, "How KV-COBRA Works": Inference, Hadamard
 *      rotation; NOVA-KV abstract: fixed per-token bit count]
 *   - decode attention: reads only the packed records; the query is projected
 *     into the key basis (q~ = P_K^T q) so keys are never reconstructed; scores
 *     s_t = scale * q~ . c^_K,t, softmax over t, o = P_V sum_t p_t c^_V,t.
 *     [KV-COBRA project page, "Efficiency": dequantization and inverse rotation
 *      in one pass over packed codes; pith.science NOVA-KV verdict, forward
 *      implications: inverse key transform folded into the query]
 *
 * Record format of one token (rank r, bits b), W = 1 + ceil(r*b/32) words:
 *   word 0      : fp16 bits of min (bits 0-15) | fp16 bits of step (bits 16-31)
 *   words 1..W-1: codes as one little-endian bitstream, bit k of code j at
 *                 stream bit j*b + k, stream bit s at bit s%32 of word 1+s/32;
 *                 codes may straddle words; unused high bits are zero.
 *   Dequantized coordinate j: min + step * code_j.
 *   Quantizer: min = fp16_rne(min_j c_j); step = fp16_rne(max(max_j c_j - min, 0)/(2^b - 1));
 *   code_j = clamp(round_half_even((c_j - min)/step), 0, 2^b - 1), all zero if step == 0.
 *   All rounding decisions are those of exact (float64) arithmetic.
 * Header-free records (a layout with static scales for that tensor): the same
 *   record without word 0, W - 1 = ceil(r*b/32) words; min and step are the
 *   head's fixed values and code_j = clamp(round_half_even((c_j - min)/step),
 *   0, 2^b - 1).  [KV-COBRA project page, "How KV-COBRA Works", Hadamard
 *   rotation: one uniform quantizer per head suffices; abstract: no per-token
 *   overhead]
 *
 * Vector-quantized records (a layout with vq_k / vq_v = 2 for that tensor): the
 *   coordinates are taken in pairs (2j, 2j+1), each pair with its own codebook
 *   of 2^b two-dimensional fp16 codewords (b index bits per pair, b/2 bits per
 *   coordinate); W = 1 + ceil((r/2)*b/32) words:
 *   word 0      : fp16 bits of +0 (bits 0-15) | fp16 bits of rho (bits 16-31),
 *                 rho = fp16_rne(sqrt(mean_j c_j^2)), the token's RMS scale;
 *   words 1..W-1: the r/2 pair indices as the bitstream above (b bits each).
 *   Reconstructed coordinates (2j, 2j+1) = rho * codebook_j[index_j]; a decoder
 *   of the scalar records therefore reads (min, step) = (0, rho).  Encode: u =
 *   c / rho (u = 0 when rho = 0), index_j = the codeword w nearest (u_2j, u_2j+1)
 *   in float64 (u_2j - w0)^2 + (u_2j+1 - w1)^2, the first one on ties.
 *   Codebook layout: per head, (r_h / 2) pairs x 2^b_h codewords of one uint32
 *   each (fp16 of the even coordinate in bits 0-15, of the odd one in bits
 *   16-31), heads concatenated.  The calibration that makes codebooks (k-means
 *   on RMS-normalised coefficient pairs, the coefficients grouped so that each
 *   pair's variance product is about equal) and orders the basis columns
 *   accordingly is the caller's.  [NOVA-KV abstract: MSE-optimal vector
 *   quantizers on the transformed coefficients, equal-volume grouping with
 *   equal-size codebooks for a fixed-width layout; pith.science NOVA-KV verdict,
 *   key_machinery and referee_report: groups dealt by log-variance, k-means
 *   codebooks on per-token RMS-normalised coefficients with a per-token scale;
 *   forward_implications: a fixed-width codebook lookup plus a per-token scale
 *   on the read path]
 *
 * Cache layout (one flat uint32 array per tensor, K and V separately):
 *   head-major regions; region h holds batch x capacity records of W_h words
 *   (one word fewer for header-free records);
 *   record (h, b, t) starts at word  sum_{h'<h} batch*capacity*W_h'  +  (b*capacity + t)*W_h.
 * Paged cache layout (page_tokens > 0): region h is a pool of pool_pages pages of
 *   page_tokens records; logical page p of sequence b is pool page
 *   P = block_table[b][p], and record (h, b, t) starts at word
 *   sum_{h'<h} pool_pages*page_tokens*W_h'  +  (P*page_tokens + t % page_tokens)*W_h
 *   with P = block_table[b][t / page_tokens].  capacity (a multiple of
 *   page_tokens) is the longest sequence; sequences may share no page (the
 *   library does not check).  A block-table entry outside [0, pool_pages) is
 *   never written through and its records read as zeros.  The block table is
 *   read by the kernels on `stream`, so earlier work on the stream may update it.
 *   [PagedAttention, cited among the pages' serving systems; the records keep
 *   their fixed width, so a page is a plain array of them]
 *
 * Basis layout: the heads' bases concatenated, head h is a row-major
 *   head_dim x r_h float32 matrix (element (i, j) at offset_h + i*r_h + j),
 *   offset_h = sum_{h'<h} head_dim * r_h'.
 *   With query_basis_k = 1 the key bases form pairs: head h's block is P_K
 *   (head_dim x r) followed by Q_K (head_dim x r), offset_h = sum_{h'<h} 2 *
 *   head_dim * r_h'.  Keys are encoded with P_K (c = P_K^T k) and reconstructed
 *   through Q_K (k^ = Q_K c^), so attention projects the query with Q_K
 *   (q . k^ = (Q_K^T q) . c^).  For an orthonormal basis Q_K = P_K.  This
 *   carries a non-orthogonal key transform: P_K = (M_q^(1/2) E)_r and Q_K =
 *   (M_q^(-1/2) E)_r with P_K^T Q_K = I.  [NOVA-KV abstract; pith.science
 *   NOVA-KV verdict, key_machinery: R_K = M_q^(1/2) E, R_K R_K^T = M_q, the
 *   inverse key transform folded into the query]
 *
 * Conventions for every call:
 *   - pointers are DEVICE memory unless the comment says HOST;
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream);
 *     every call only enqueues work on it, never synchronizes, never allocates
 *     or frees device memory, and keeps no state between calls;
 *   - the caller owns every buffer; the library keeps no pointer after return;
 *   - arguments are validated on the host before anything is launched; on
 *     failure nothing is launched, a non-zero kv_status is returned and
 *     kv_last_error() describes the problem (the message is thread-local);
 *   - launch failures return KV_ERR_DEVICE; kernel faults surface at the
 *     caller's next synchronization, as with any HIP work.
 *   - supported: head_dim = 128, rank in {16, 32, 64, 128}, bits in [2, 8],
 *     1 <= n_kv_heads <= 64, n_q_heads = g * n_kv_heads with 1 <= g <= 16.
 */
#ifndef KVTC_H
#define KVTC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_status {
  KV_OK = 0,
  KV_ERR_INVALID = 1,     /* null pointer, bad shape, misalignment, buffer too small */
  KV_ERR_UNSUPPORTED = 2, /* head_dim, rank, bits or head counts outside the supported set */
  KV_ERR_CAPACITY = 3,    /* token positions beyond the cache capacity */
  KV_ERR_DEVICE = 4       /* a HIP runtime call or kernel launch failed */
} kv_status;

typedef enum kv_dtype { KV_F32 = 0, KV_F16 = 1 } kv_dtype;

/* Shape and per-head allocation of one layer's compressed cache.  The
 * allocation and scale arrays are HOST memory with n_kv_heads entries each;
 * they are read during the call only.  Query head h' reads KV head h'/g (g =
 * n_q_heads / n_kv_heads, contiguous groups).  Per-head (rank, bits) is the
 * allocation a calibration step (for example the C1 search of the KV-COBRA
 * page) chose; the library takes it as given.  scale_k / scale_v: NULL for
 * records with per-token headers, else the head's fixed quantizer for
 * header-free records of that tensor, fp16 bits of min | fp16 bits of step
 * << 16 (finite, step > 0), also chosen at calibration.  Vector-quantized
 * records (vq_k / vq_v) keep their per-token scale word, so they take no static
 * scale; decode attention runs them in the kernel classes compiled for their
 * formats (rank 32, 64 or 128 with 2-8 index bits, listed in the class table of
 * the library) and returns KV_ERR_UNSUPPORTED for others. */
typedef struct kv_layout {
  int32_t head_dim;       /* d; must be 128 */
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t batch;
  int64_t capacity;       /* records per sequence and head; > 0 */
  const int32_t *rank_k;  /* HOST [n_kv_heads] */
  const int32_t *bits_k;  /* HOST [n_kv_heads] */
  const int32_t *rank_v;  /* HOST [n_kv_heads] */
  const int32_t *bits_v;  /* HOST [n_kv_heads] */
  const uint32_t *scale_k; /* HOST [n_kv_heads] or NULL */
  const uint32_t *scale_v; /* HOST [n_kv_heads] or NULL */
  int32_t query_basis_k;   /* 0: orthonormal key bases; 1: each head's key basis block holds
                              the encode basis P_K then the query basis Q_K (see below) */
  int32_t page_tokens;     /* 0: each sequence's records contiguous (see the cache layout);
                              > 0: paged records, pages of this many tokens (a multiple of 64) */
  int64_t pool_pages;      /* paged: pages in each head's pool */
  const int32_t *block_table; /* paged: DEVICE int32 [batch][capacity / page_tokens], the pool
                              page holding each logical page of each sequence */
  int32_t vq_k;            /* 0: scalar-quantized K records; 2: vector-quantized K records over
                              coordinate pairs (bits_k = index bits per pair, see above) */
  int32_t vq_v;            /* the same for V */
  const uint32_t *codebook_k; /* vq_k = 2: DEVICE K codebooks (layout above), else NULL */
  const uint32_t *codebook_v; /* vq_v = 2: DEVICE V codebooks, else NULL */
} kv_layout;

/* Words per record with its header, 1 + ceil(rank*bits/32) (a header-free
 * record has one word fewer); 0 if (rank, bits) is unsupported. */
int32_t kv_record_words(int32_t rank, int32_t bits);

/* Bytes of the K (which = 0) or V (which = 1) cache of `layout`, written to *bytes (HOST). */
kv_status kv_cache_bytes(const kv_layout *layout, int32_t which, size_t *bytes);

/* Bytes of device workspace kv_attend_decode needs for n_tokens context tokens. */
kv_status kv_workspace_bytes(const kv_layout *layout, int64_t n_tokens, size_t *bytes);

/* How decode attention over `layout` runs, written to HOST ints (any may be NULL):
 * kernel_class: -1 for the generic kernel (widths read at run time), 0..6 for the
 * built-in classes (0-3: the formats of one per-vector budget of 64, 128, 256, 512
 * bits with per-token headers; 4-5: 64, 128 bits header-free; 6: vector-quantized
 * pairs), 7 and up for the classes the build compiled from frozen layer
 * allocations, in the order they are listed; splits: the largest number of splits
 * of one (sequence, KV head) for n_tokens and split_tokens (0: the default plan);
 * workgroups: the launch's grid size.  No device work.  Errors as
 * kv_workspace_bytes_split, and KV_ERR_UNSUPPORTED for vector-quantized formats
 * no class holds. */
kv_status kv_attend_plan(const kv_layout *layout, int64_t n_tokens, int64_t split_tokens,
                         int32_t *kernel_class, int32_t *splits, int32_t *workgroups);

/* Prefill encode.  k, v: [batch][n_kv_heads][n_tokens][head_dim] of `dtype`
 * (KV_F32 or KV_F16), contiguous, 16-byte aligned when n_tokens > 1; every
 * token must have ||x||_2 * max_j ||P_j||_2 <= 65504 (its coordinates, bounded by
 * that product, then keep the fp16 min and step finite; an orthonormal basis has
 * unit columns; outside that range the records are unspecified but the call stays
 * defined).
 * Writes records
 * pos0 .. pos0+n_tokens-1 of every (sequence, head) into cache_k / cache_v
 * (other records untouched).  basis_k / basis_v: concatenated float32 bases
 * (layout above).  The projection runs on the matrix cores; every rounding
 * decision it cannot settle within its error bound is taken from the float64
 * projection, so the records are those of kv_append token by token.
 * Errors: KV_ERR_CAPACITY if pos0 < 0 or pos0 + n_tokens > capacity;
 * KV_ERR_INVALID for misaligned inputs; n_tokens == 0 launches nothing and
 * returns KV_OK.
 * [KV-COBRA project page, "How KV-COBRA Works", Inference; the projection
 *  d -> r is a dense T x d by d x r contraction per head] */
kv_status kv_encode(const kv_layout *layout, const void *k, const void *v, kv_dtype dtype,
                    int64_t n_tokens, int64_t pos0, const float *basis_k, const float *basis_v,
                    uint32_t *cache_k, uint32_t *cache_v, void *stream);

/* Decode-time append of one token per (sequence, head) at position `pos`.
 * k1, v1: [batch][n_kv_heads][head_dim] of `dtype`.  Same arithmetic and
 * records as kv_encode with n_tokens = 1. */
kv_status kv_append(const kv_layout *layout, const void *k1, const void *v1, kv_dtype dtype,
                    int64_t pos, const float *basis_k, const float *basis_v,
                    uint32_t *cache_k, uint32_t *cache_v, void *stream);

/* Decode attention of one query per (sequence, query head) over records
 * 0 .. n_tokens-1 of every sequence.
 *   q:   [batch][n_q_heads][head_dim] of `dtype` (KV_F32 or KV_F16)
 *   out: [batch][n_q_heads][head_dim] float32, fully overwritten
 *   softmax_scale: multiplies q . k (1/sqrt(head_dim) for standard attention)
 *   workspace: at least kv_workspace_bytes(layout, n_tokens) bytes, 16-byte
 *              aligned, caller-owned.  Its first 4 * batch * n_kv_heads bytes
 *              are split arrival counters, one per (sequence, KV head): zero-fill
 *              a new workspace (and again after using it for anything else);
 *              every completed call leaves them zero.  The rest is scratch whose
 *              contents on entry are ignored.  A counter that is not zero on
 *              entry (a workspace that was not zero-filled, or one left by an
 *              aborted launch) never makes the output wrong: every split
 *              partial carries a tag of the call that wrote it, and a merge
 *              that would fold a partial this call has not written writes NaN
 *              instead, so that unit's output elements are each either NaN or
 *              the correct value.  A counter at or above the unit's split count
 *              is not reset by the call.  Calls that share a workspace must not
 *              overlap in time.
 * n_tokens == 0 writes zeros to `out`.  Errors: KV_ERR_CAPACITY if
 * n_tokens > capacity; KV_ERR_INVALID if the workspace is too small.
 * [KV-COBRA project page, "Efficiency"; pith.science NOVA-KV verdict,
 *  forward implications] */
kv_status kv_attend_decode(const kv_layout *layout, const void *q, kv_dtype dtype, int64_t n_tokens,
                           const float *basis_k, const float *basis_v, const uint32_t *cache_k,
                           const uint32_t *cache_v, float softmax_scale, float *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* As kv_attend_decode with an explicit split-K size (a positive multiple of
 * 256; 0 picks the default).  The context of every (sequence, KV head) is cut
 * into ns = ceil(n_tokens / split_tokens) splits of whole 256-token blocks:
 * with nq = ceil(n_tokens / 256) blocks, split x takes blocks [q(x), q(x+1))
 * where q(x) = min(nq, floor(x * (nq + e) / ns)) and e = min(8, max(2,
 * floor(nq / (2 ns)))).  Consecutive splits differ by at most one block, and
 * the last splits are about e blocks lighter (the newest token's split also
 * encodes it in kv_append_attend_decode); with few
 * blocks per split a split may be larger than split_tokens and the last ones
 * may be empty (n_tokens = 512, split_tokens = 256: 512 and 0 tokens).  The
 * default fills every resident workgroup slot of the GPU, with at most
 * floor(n_tokens / 1024) splits per unit (shorter splits cost more in per-split
 * fixed work than they gain in parallelism; 32769 tokens take 32 splits, not 33),
 * giving each KV head a number of splits in proportion to the cost
 * of its tokens (record words per token, key plus value, plus a fixed per-token
 * share for the softmax), so that heads of different widths finish together.
 * The result is the same up to float rounding for every split size.  The
 * workspace must hold kv_workspace_bytes_split(layout, n_tokens, split_tokens)
 * bytes. */
kv_status kv_workspace_bytes_split(const kv_layout *layout, int64_t n_tokens, int64_t split_tokens,
                                   size_t *bytes);
kv_status kv_attend_decode_split(const kv_layout *layout, const void *q, kv_dtype dtype,
                                 int64_t n_tokens, int64_t split_tokens, const float *basis_k,
                                 const float *basis_v, const uint32_t *cache_k,
                                 const uint32_t *cache_v, float softmax_scale, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Decode attention over sequences of different lengths: sequence b attends over
 * its tokens 0 .. lengths[b]-1.  lengths: DEVICE int32 [batch], read by the
 * kernel on `stream` (so it can be written by earlier work on that stream), each
 * value clamped to [0, max_tokens]; max_tokens <= capacity sets the split plan
 * and the workspace size (kv_workspace_bytes(layout, max_tokens)).  A sequence
 * of length 0 gets an all-zero output.  Otherwise as kv_attend_decode.  Errors
 * as kv_attend_decode, plus KV_ERR_INVALID for a NULL or misaligned lengths.
 * [KV-COBRA project page, "Efficiency" (the decode attention over the packed
 *  cache), for a batch of requests at different positions] */
kv_status kv_attend_decode_ragged(const kv_layout *layout, const void *q, kv_dtype dtype,
                                  const int32_t *lengths, int64_t max_tokens, const float *basis_k,
                                  const float *basis_v, const uint32_t *cache_k, const uint32_t *cache_v,
                                  float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* One decode step in one launch: append the new token of every (sequence, head)
 * at position n_tokens - 1, then attend over records 0 .. n_tokens-1, the new
 * one included.  k1, v1: [batch][n_kv_heads][head_dim] of `kv_dt` (KV_F32 or
 * KV_F16); the other arguments, the workspace contract and the result are those
 * of kv_attend_decode_split.  The records written are bit-identical to those of
 * kv_append(pos = n_tokens - 1) and `out` equals that of kv_append followed by
 * kv_attend_decode_split with the same split size: the workgroup whose split
 * holds the new position encodes it before it reads that split.
 * Errors: KV_ERR_INVALID if n_tokens < 1 or k1 / v1 is NULL; otherwise as
 * kv_attend_decode_split.
 * [KV-COBRA project page, "How KV-COBRA Works", Inference (each new key and
 *  value is compressed as it is produced) and "Efficiency"] */
kv_status kv_append_attend_decode(const kv_layout *layout, const void *k1, const void *v1,
                                  kv_dtype kv_dt, const void *q, kv_dtype q_dt,
                                  int64_t n_tokens, int64_t split_tokens, const float *basis_k,
                                  const float *basis_v, uint32_t *cache_k, uint32_t *cache_v,
                                  float softmax_scale, float *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* kv_append_attend_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that must
 * not allocate, harnesses that forbid it).  The split counters and partials live
 * in a static device array of the library, 16 MiB per GPU (held until the
 * process ends): its first 4096 words are arrival counters, the rest partials.
 * The call itself calls no allocating routine.  Arguments, records and output
 * are those of kv_append_attend_decode with the same split size.
 * The counters are zero when the library's code loads on a device and every
 * completed call leaves them zero; a counter that is not (a launch that did not
 * complete) gives NaN or correct outputs, as for kv_attend_decode.  Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on different streams, or from several threads) race and must not be issued.
 * `stream` must belong to the current device.
 * Errors: KV_ERR_CAPACITY if batch * n_kv_heads > 4096 or the split partials
 * (4 * 132 bytes per sequence, query head and split) exceed 16 MiB - 16 KiB;
 * KV_ERR_INVALID if `stream` is on another device; otherwise as
 * kv_append_attend_decode. */
kv_status kv_append_attend_decode_noalloc(const kv_layout *layout, const void *k1, const void *v1,
                                          kv_dtype kv_dt, const void *q, kv_dtype q_dt,
                                          int64_t n_tokens, int64_t split_tokens, const float *basis_k,
                                          const float *basis_v, uint32_t *cache_k, uint32_t *cache_v,
                                          float softmax_scale, float *out, void *stream);

/* Decode attention over keys compressed before the rotary position embedding
 * (RoPE): the cache holds the codes of each token's unrotated key (as kv_encode
 * and kv_append write them from pre-RoPE keys), and the score of token t is
 *     s_t = softmax_scale * q . RoPE(k^_t, t),   k^_t = Q_K (min_t + step_t code_t),
 * with Q_K the head's key reconstruction basis (P_K, or the query-side basis of a
 * query_basis_k layout).  RoPE turns each dimension pair (2i, 2i+1) of a vector at
 * position t by the angle t * inv_freq[i]; token t of a sequence sits at position
 * t.  q: [batch][n_q_heads][128] of `dtype`, already rotated to its own position.
 * inv_freq: DEVICE float64 [64] (RoFormer's base^(-2i/128), or any other
 * frequencies; a model that pairs dimensions (i, i + 64) is this rotation after a
 * fixed permutation of the head dimensions, applied to its keys, queries and
 * bases).  Values, softmax, splits, merges and the workspace contract are those
 * of kv_attend_decode_split, but the split plan is this kernel's own: the
 * workspace must hold kv_workspace_bytes_rope(layout, n_tokens, split_tokens)
 * bytes.  Each key is reconstructed in the head dimension on the matrix cores
 * (2 * 128 * r_K products per token): wide keys make this path bound by
 * arithmetic rather than by the cache bytes.
 * Errors: KV_ERR_UNSUPPORTED for vector-quantized records or a group of more
 * than 8 query heads; KV_ERR_INVALID for a NULL or misaligned inv_freq; otherwise
 * as kv_attend_decode_split.
 * [KV-COBRA project page, Results (the note under the results table: keys
 *  compressed before RoPE); rotary embedding as defined by RoFormer] */
kv_status kv_workspace_bytes_rope(const kv_layout *layout, int64_t n_tokens, int64_t split_tokens,
                                  size_t *bytes);
kv_status kv_attend_decode_rope(const kv_layout *layout, const void *q, kv_dtype dtype, int64_t n_tokens,
                                int64_t split_tokens, const float *basis_k, const float *basis_v,
                                const uint32_t *cache_k, const uint32_t *cache_v, float softmax_scale,
                                const double *inv_freq, float *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* kv_append_attend_decode for keys compressed before RoPE: appends the new
 * (unrotated) key and value at position n_tokens - 1, then attends as
 * kv_attend_decode_rope.  The records are those of kv_append; `out` equals that of
 * kv_append followed by kv_attend_decode_rope with the same split size.  Errors
 * as kv_append_attend_decode and kv_attend_decode_rope. */
kv_status kv_append_attend_decode_rope(const kv_layout *layout, const void *k1, const void *v1,
                                       kv_dtype kv_dt, const void *q, kv_dtype q_dt, int64_t n_tokens,
                                       int64_t split_tokens, const float *basis_k, const float *basis_v,
                                       uint32_t *cache_k, uint32_t *cache_v, float softmax_scale,
                                       const double *inv_freq, float *out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Reconstruct stored tokens: for records pos0 .. pos0+n_tokens-1 of every
 * (sequence, KV head) of tensor `which` (0 = K, 1 = V), x^ = B (min + step *
 * code) with B that head's reconstruction basis (`basis`: the tensor's
 * concatenated bases; B = P, or Q_K for the keys of a query_basis_k layout),
 * each coordinate dequantized exactly and the d outputs summed in float32 over
 * the coordinates in order.  out: DEVICE float32 [batch][n_kv_heads][n_tokens]
 * [head_dim].  Not on the decode path (attention reads the codes directly):
 * for measuring distortion and for consumers that need the vectors.
 * Errors: KV_ERR_CAPACITY if pos0 < 0 or pos0 + n_tokens > capacity;
 * KV_ERR_INVALID for NULL or misaligned pointers or which outside {0, 1};
 * n_tokens == 0 launches nothing.
 * [KV-COBRA project page, "How KV-COBRA Works", Inference: the inverse of the
 *  rotation and truncation] */
kv_status kv_decode(const kv_layout *layout, int32_t which, int64_t n_tokens, int64_t pos0,
                    const float *basis, const uint32_t *cache, float *out, void *stream);

/* Quantize and pack n tokens of r float32 coordinates each (coords [n][r])
 * into records [n][kv_record_words(r, b)].  Same device code as the encoder's
 * quantize/pack stage; exposed to check the record format in isolation. */
kv_status kv_quantize_pack(const float *coords, int64_t n, int32_t rank, int32_t bits,
                           uint32_t *records, void *stream);

/* Inverse of the packing: records [n][W] -> min_step [n][2] (fp16 bit
 * patterns of min and step) and codes [n][rank] (uint8).  Uses the decode
 * kernels' unpack routines. */
kv_status kv_unpack(const uint32_t *records, int64_t n, int32_t rank, int32_t bits,
                    uint16_t *min_step, uint8_t *codes, void *stream);

/* Message describing the last failed call on this thread ("" if none). */
const char *kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVTC_H */
