// Shared host/device definitions of the kvtc library (gfx950).
//
// Record format, quantizer and cache layout are documented in include/kvtc.h.
// Everything here is written for CDNA4: 64-wide wavefronts, fp64 at full
// VALU rate for the exact rounding decisions of the quantizer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvtc {

constexpr int kHeadDim = 128;     // supported head dimension
constexpr int kMaxKvHeads = 64;   // KV heads per layout (kernel-argument table size)
constexpr int kMaxGroup = 16;     // query heads per KV head
constexpr int kMaxRank = 128;
constexpr int kMinBits = 2;
constexpr int kMaxBits = 8;
constexpr int kMaxWords = 1 + (kMaxRank * kMaxBits + 31) / 32;  // 33
constexpr int kSplitQuantum = 256;  // split-K sizes are multiples of this
constexpr int kPartStride = 132;    // floats per split partial: o[128], m, l, tag, pad

__host__ __device__ inline int record_words(int r, int b) { return 1 + (r * b + 31) / 32; }
// Words of a record with (hdr = 1) or without (hdr = 0) its per-token header word.
__host__ __device__ inline int record_words(int r, int b, int hdr) { return hdr + (r * b + 31) / 32; }

// Record formats are named by a width code B: 2..8 for b-bit scalar codes, kVq + b
// for vector-quantized records of coordinate pairs with b-bit indices (one index per
// pair; the codebook entry of pair j holds fp16 coordinates 2j and 2j + 1).
constexpr int kVq = 16;
__host__ __device__ constexpr bool is_vq(int B) { return B >= kVq; }
__host__ __device__ constexpr int code_bits(int B) { return B >= kVq ? B - kVq : B; }
__host__ __device__ constexpr int code_count(int r, int B) { return B >= kVq ? r / 2 : r; }
// Words of a record of rank r in format B, with or without the header word.
__host__ __device__ inline int format_words(int r, int B, int hdr) {
  return hdr + (code_count(r, B) * code_bits(B) + 31) / 32;
}
// 32-bit codebook entries of a vector-quantized tensor of rank r (r/2 pairs x 2^b).
__host__ __device__ inline int codebook_words(int r, int B) { return is_vq(B) ? (r / 2) << code_bits(B) : 0; }

// LDS row stride (words) of the per-pair codebooks in the decode kernel.  Keys: the
// four lane groups of a score operand read pairs 4 * nks apart (nks = r/32 K-steps),
// so with at most 16 entries per pair the stride is padded until those reads fall in
// four different quarters of the 64 LDS banks; values: an odd stride spreads the
// sixteen pairs one operand reads over the banks.
__host__ __device__ constexpr int vq_kstride(int B, int r) {
  const int e = 1 << code_bits(B), nks = r >= 32 ? r / 32 : 1;
  if (e <= 16)
    for (int pad = 0; pad < 16; ++pad)
      if ((4 * nks * (e + pad)) % 64 == 16) return e + pad;
  return e + 1;
}
__host__ __device__ constexpr int vq_vstride(int B) { return (1 << code_bits(B)) + 1; }
// LDS words of a head's codebooks in the decode kernel (keys then values).
__host__ __device__ inline int vq_lds_words(int rk, int bk, int rv, int bv) {
  return (is_vq(bk) ? (rk / 2) * vq_kstride(bk, rk) : 0) + (is_vq(bv) ? (rv / 2) * vq_vstride(bv) : 0);
}

inline bool supported_rank(int r) { return r == 16 || r == 32 || r == 64 || r == 128; }
inline bool supported_bits(int b) { return b >= kMinBits && b <= kMaxBits; }

// Per-KV-head allocation and addressing, passed by value in kernel arguments
// (56 bytes: 64 heads of it fit the 4 KB argument segment with the rest).
struct HeadDesc {
  int64_t base_k, base_v;   // word offset of the head's cache region
  int32_t boff_k, boff_v;   // float offset of the head's (encode) basis
  int32_t qoff_k;           // float offset of the head's query-side key basis (== boff_k when orthonormal)
  uint32_t sk, sv;          // header-free records: the head's fixed fp16 min | fp16 step << 16;
                            // vector-quantized records: the word offset of the head's codebook
  int32_t ns;               // splits of each of the head's (sequence, head) units (set at launch)
  int16_t wk, wv;           // record words
  int16_t spec;             // index of the format in the specialised kernel's class (set at launch)
  uint8_t rk, bk, rv, bv;   // rank and format code B (bits, or kVq + index bits) of keys and values
  uint8_t hk, hv;           // header words of a key / value record: 1 (per-token min and step) or 0
};
static_assert(sizeof(HeadDesc) == 56, "HeadDesc layout");

struct HeadTable {
  HeadDesc h[kMaxKvHeads];
};

// Head h's descriptor from a kernel-argument table, read as 32-bit words: a
// uniform h makes them scalar loads, issued together (one round trip), where the
// 8- and 16-bit fields read in place would each be a vector load of its own.
__device__ inline HeadDesc head_desc(const HeadTable& t, int h) {
  struct Words {
    uint32_t w[sizeof(HeadDesc) / 4];
  } x;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(&t.h[h]);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(HeadDesc) / 4); ++i) x.w[i] = p[i];
  return __builtin_bit_cast(HeadDesc, x);
}

// Where the records of a sequence live within its head's cache region: contiguous
// (bt == null: token t of sequence b is record b * capacity + t) or paged (token t
// in pool page bt[b * pages_per_seq + t / page], slot t % page; the region is the
// head's pool of pool_pages pages).
struct Paging {
  const int32_t* bt;      // DEVICE [batch][pages_per_seq] block table, or null
  int32_t page;           // tokens per page (a multiple of 64)
  int32_t pages_per_seq;  // capacity / page
  int64_t pool_pages;     // pages in each head's pool
};

// Record index of token t of sequence b in its head's region, or -1 when the block
// table names a page outside the pool (nothing is written there; reads see zeros).
__device__ inline int64_t record_index(const Paging& pg, int64_t capacity, int b, int64_t t) {
  if (!pg.bt) return (int64_t)b * capacity + t;
  const int64_t p = pg.bt[(int64_t)b * pg.pages_per_seq + t / pg.page];
  if (p < 0 || p >= pg.pool_pages) return -1;
  return p * pg.page + t % pg.page;
}

// ------------------------------------------------------------------ fp16 helpers
// Round a double to the nearest binary16 (ties to even) in one step, returning
// the bit pattern.  Handles subnormal results, overflow to infinity and NaN.
__device__ inline uint32_t f64_to_f16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return sign | 0x7C00u | (a > 0x7FF0000000000000ull ? 0x200u : 0u);
  if (a < 0x0010000000000000ull) return sign;  // zero or double subnormal
  int e = (int)(a >> 52) - 1023;
  if (e < -25) return sign;
  if (e > 15) return sign | 0x7C00u;
  uint64_t m = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
  int shift = (e >= -14) ? 42 : 28 - e;  // low bits of the 53-bit significand to drop
  uint64_t keep = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1ull);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1ull))) keep++;
  if (e >= -14) {
    int E = e + 15;
    if (keep == 2048ull) { keep = 1024ull; E++; }
    if (E >= 31) return sign | 0x7C00u;
    return sign | ((uint32_t)E << 10) | (uint32_t)(keep & 0x3FFull);
  }
  return sign | (uint32_t)keep;  // subnormal (keep == 1024 encodes the smallest normal)
}

__device__ inline float f16_bits_to_f32(uint32_t bits) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
  return (float)h;
}

__device__ inline double f16_bits_to_f64(uint32_t bits) { return (double)f16_bits_to_f32(bits); }

// ------------------------------------------------------------------ quantizer
// Header of one token from its exact coordinate extremes (float64 semantics):
// min = fp16(cmin); step = fp16(max(cmax - min, 0) / (2^b - 1)).
struct QuantHeader {
  uint32_t word0;  // fp16(min) | fp16(step) << 16
  double mu, sigma;
};

// The header of a head whose quantizer is fixed (header-free records).
__device__ inline QuantHeader static_header(uint32_t word0) {
  QuantHeader q;
  q.word0 = word0;
  q.mu = f16_bits_to_f64(word0 & 0xFFFFu);
  q.sigma = f16_bits_to_f64(word0 >> 16);
  return q;
}

__device__ inline QuantHeader quant_header(double cmin, double cmax, int b) {
  QuantHeader q;
  uint32_t mb = f64_to_f16_rne(cmin);
  q.mu = f16_bits_to_f64(mb);
  double range = cmax - q.mu;
  if (!(range > 0.0)) range = 0.0;
  uint32_t sb = f64_to_f16_rne(range / (double)((1 << b) - 1));
  q.sigma = f16_bits_to_f64(sb);
  q.word0 = mb | (sb << 16);
  return q;
}

// code = clamp(rint((c - mu) / sigma), 0, 2^b - 1), all zero when sigma == 0.
// An undefined argument (NaN: only for inputs beyond the supported range, whose
// fp16 min or step overflowed) gives code 0 rather than a NaN-to-integer cast.
__device__ inline uint32_t quant_code(double c, double mu, double sigma, int b) {
  if (!(sigma > 0.0)) return 0u;
  double u = __builtin_rint((c - mu) / sigma);
  double top = (double)((1 << b) - 1);
  u = !(u > 0.0) ? 0.0 : (u > top ? top : u);
  return (uint32_t)u;
}

// Word w (0-based among the code words) of the little-endian code stream,
// gathered from codes[0..r) held in LDS (32-bit or 8-bit code elements).
template <typename C>
__device__ inline uint32_t pack_word(const C* codes, int r, int b, int w) {
  const int lo = 32 * w;
  int j0 = lo / b;
  int j1 = (lo + 31) / b;
  if (j1 > r - 1) j1 = r - 1;
  uint32_t word = 0u;
  for (int j = j0; j <= j1; ++j) {
    int off = j * b - lo;
    uint32_t c = (uint32_t)codes[j];
    word |= off >= 0 ? (c << off) : (c >> (-off));
  }
  return word;
}

// Code j of a record whose code words start at `words` (generic b, may straddle).
__device__ inline uint32_t unpack_code(const uint32_t* words, int j, int b) {
  int bit = j * b;
  int w = bit >> 5, off = bit & 31;
  uint32_t v = words[w] >> off;
  if (off + b > 32) v |= words[w + 1] << (32 - off);
  return v & ((1u << b) - 1u);
}

}  // namespace kvtc
