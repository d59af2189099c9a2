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
constexpr int kPartStride = 132;    // floats per split partial: m, l, o~[128], pad

__host__ __device__ inline int record_words(int r, int b) { return 1 + (r * b + 31) / 32; }

inline bool supported_rank(int r) { return r == 16 || r == 32 || r == 64 || r == 128; }
inline bool supported_bits(int b) { return b >= kMinBits && b <= kMaxBits; }

// Per-KV-head allocation and addressing, passed by value in kernel arguments.
struct HeadDesc {
  int32_t rk, bk, rv, bv;   // rank and bits of keys and values
  int32_t wk, wv;           // record words
  int32_t boff_k, boff_v;   // float offset of the head's basis
  int64_t base_k, base_v;   // word offset of the head's cache region
  int32_t spec;             // index of the format in the specialised kernel's class (set at launch)
  int32_t ns;               // splits of each of the head's (sequence, head) units (set at launch)
};

struct HeadTable {
  HeadDesc h[kMaxKvHeads];
};

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
__device__ inline uint32_t quant_code(double c, double mu, double sigma, int b) {
  if (!(sigma > 0.0)) return 0u;
  double u = __builtin_rint((c - mu) / sigma);
  double top = (double)((1 << b) - 1);
  u = u < 0.0 ? 0.0 : (u > top ? top : u);
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
