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
 *
 * Cache layout (one flat uint32 array per tensor, K and V separately):
 *   head-major regions; region h holds batch x capacity records of W_h words;
 *   record (h, b, t) starts at word  sum_{h'<h} batch*capacity*W_h'  +  (b*capacity + t)*W_h.
 *
 * Basis layout: the heads' bases concatenated, head h is a row-major
 *   head_dim x r_h float32 matrix (element (i, j) at offset_h + i*r_h + j),
 *   offset_h = sum_{h'<h} head_dim * r_h'.
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

/* Shape and per-head allocation of one layer's compressed cache.  The four
 * allocation arrays are HOST memory with n_kv_heads entries each; they are
 * read during the call only.  Query head h' reads KV head h'/g (g =
 * n_q_heads / n_kv_heads, contiguous groups).  Per-head (rank, bits) is the
 * allocation a calibration step (for example the C1 search of the KV-COBRA
 * page) chose; the library takes it as given. */
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
} kv_layout;

/* Words per record, 1 + ceil(rank*bits/32); 0 if (rank, bits) is unsupported. */
int32_t kv_record_words(int32_t rank, int32_t bits);

/* Bytes of the K (which = 0) or V (which = 1) cache of `layout`, written to *bytes (HOST). */
kv_status kv_cache_bytes(const kv_layout *layout, int32_t which, size_t *bytes);

/* Bytes of device workspace kv_attend_decode needs for n_tokens context tokens. */
kv_status kv_workspace_bytes(const kv_layout *layout, int64_t n_tokens, size_t *bytes);

/* Prefill encode.  k, v: [batch][n_kv_heads][n_tokens][head_dim] of `dtype`
 * (KV_F32 or KV_F16), contiguous, 16-byte aligned when n_tokens > 1; float32
 * inputs must lie inside the fp16 range (|x| < 65504).  Writes records
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
 *              are split arrival counters: they must be zero before the first
 *              call (zero-fill a new workspace, and again after using it for
 *              anything else) and every completed call leaves them zero; the
 *              rest is scratch whose contents on entry are ignored.  Calls that
 *              share a workspace must not overlap in time.
 * n_tokens == 0 writes zeros to `out`.  Errors: KV_ERR_CAPACITY if
 * n_tokens > capacity; KV_ERR_INVALID if the workspace is too small.
 * [KV-COBRA project page, "Efficiency"; pith.science NOVA-KV verdict,
 *  forward implications] */
kv_status kv_attend_decode(const kv_layout *layout, const void *q, kv_dtype dtype, int64_t n_tokens,
                           const float *basis_k, const float *basis_v, const uint32_t *cache_k,
                           const uint32_t *cache_v, float softmax_scale, float *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* As kv_attend_decode with an explicit maximum number of context tokens per
 * split-K work unit (a positive multiple of 256; 0 picks the default): the
 * context of every KV head is divided into ceil(n_tokens / split_tokens)
 * splits of whole 256-token blocks whose sizes differ by at most one block.
 * The default gives each KV head a number of splits in proportion to the
 * cost of its tokens (record words per token, key plus value, plus a fixed
 * per-token share for the softmax), so that heads of different widths finish
 * together.  The result is the same up to float rounding for every
 * split size.  The workspace must
 * hold kv_workspace_bytes_split(layout, n_tokens, split_tokens) bytes. */
kv_status kv_workspace_bytes_split(const kv_layout *layout, int64_t n_tokens, int64_t split_tokens,
                                   size_t *bytes);
kv_status kv_attend_decode_split(const kv_layout *layout, const void *q, kv_dtype dtype,
                                 int64_t n_tokens, int64_t split_tokens, const float *basis_k,
                                 const float *basis_v, const uint32_t *cache_k,
                                 const uint32_t *cache_v, float softmax_scale, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream);

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

kv_status kv_append_attend_decode(const kv_layout *layout, const void *k1, const void *v1,
                                  kv_dtype kv_dt, const void *q, kv_dtype q_dt,
                                  int64_t n_tokens, int64_t split_tokens, const float *basis_k,
                                  const float *basis_v, uint32_t *cache_k, uint32_t *cache_v,
                                  float softmax_scale, float *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

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
