// Split-K decode attention over packed records on CDNA4 matrix cores (gfx950).
//
// The decode step contracts every token's codes with the g query heads of its
// KV head twice:  scores s[h, t] = q~_h . code_t  (r_K per token)  and the value
// sum  o~[h, j] = sum_t (p[h, t] step_t) code[t, j]  (r_V per token).  With g
// heads sharing one pass over the records (GQA) these are dense g x r x T
// contractions; on MI355X the fp32 VALU cannot keep up with HBM for b <= 4
// (4..6 VALU ops per code against ~4.9 lane-ops per HBM byte), so both run on
// v_mfma_f32_16x16x32_f16 and the VALU only unpacks codes and runs the softmax.
//
// Code -> fp16 operand without conversion: a b-bit code sitting at bit o <= 10-b
// of a 16-bit half is the fp16 subnormal  code * 2^(o-24); masking a 32-bit word
// with the field of the same offset in both halves yields two operands in one
// VALU op.  The matrix cores take subnormal fp16 inputs exactly, and the 2^(o-24)
// factor is folded into the other operand (keys) or the partial (values).
//
// Precision: q~ and p*step are split into fp16 hi + lo parts (two MFMAs each), so
// products carry ~22 significant bits and accumulate in fp32.
//
// Pages: KV-COBRA project page, "Efficiency" (dequantization and inverse rotation
// in one pass over packed codes); pith.science NOVA-KV verdict, forward
// implications (the inverse key transform folded into the query).
#include "kvtc_common.h"
#include "kvtc_launch.h"

namespace kvtc {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));  // records are 4-byte aligned
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kTileT = 64;      // tokens per wave iteration
constexpr int kWaveLds = 2048;  // 32-bit words of LDS per wave (scores, probabilities, partial)

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ inline uint32_t h2u(_Float16 x) { return (uint32_t)__builtin_bit_cast(uint16_t, x); }

__device__ inline void lds_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

__device__ inline float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}


__device__ inline float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ----------------------------------------------------------------- buffer loads
// One buffer resource per (sequence, KV head) cache region: 32-bit byte offsets,
// loads past the region return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint32_t ld16(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ inline uint32_t ld32(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0); }
__device__ inline u32x2 ld64(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0); }
__device__ inline u32x4 ld128(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0); }

template <int N>
__device__ inline void load_words(rsrc_t r, uint32_t off, uint32_t (&w)[N]) {
  if constexpr (N == 1) {
    w[0] = ld32(r, off);
  } else if constexpr (N == 2) {
    const u32x2 a = ld64(r, off);
    w[0] = a[0]; w[1] = a[1];
  } else {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      const u32x4 a = ld128(r, off + 4 * k);
      w[k] = a[0]; w[k + 1] = a[1]; w[k + 2] = a[2]; w[k + 3] = a[3];
    }
  }
}

// Adjacent codes at stream bit `bit` (general widths): low code in bits 0..B-1.
__device__ inline uint32_t window(rsrc_t r, uint32_t rec_off, int bit) {
  const u32x2 a = ld64(r, rec_off + 4u * (1 + (bit >> 5)));
  return __builtin_amdgcn_alignbit(a[1], a[0], bit & 31);
}

// ----------------------------------------------------------------- code fields
// Power-of-two widths (2, 4, 8): a pair operand holds the codes at the same
// offset of the two 16-bit halves of a word; offsets whose field would reach the
// fp16 exponent bits (10..14) are taken after a pre-shift of kShift bits.
template <int B> struct Pow2 {
  static constexpr int kPerHalf = 16 / B;
  static constexpr int kShift = (B == 2) ? 10 : 8;
  static constexpr uint32_t kMask = (1u << B) - 1u;
  __device__ static constexpr int pre(int o) { return (o + B <= 10) ? 0 : kShift; }
  __device__ static constexpr int at(int o) { return o - pre(o); }
  __device__ static inline uint32_t pair(uint32_t y, int o) {
    return (y >> pre(o)) & ((kMask << at(o)) | (kMask << (16 + at(o))));
  }
};

__host__ __device__ constexpr bool pow2_bits(int b) { return b == 2 || b == 4 || b == 8; }

// Key pair slots.  Lane group G of a 16-token sub-tile owns pair slots
// [G*nks*4, (G+1)*nks*4) of its token (nks = max(1, r_K/32) K-steps of 32 codes).
// Power-of-two widths: pair pi = the codes at half-offset (pi % (16/B))*B of code
// word pi / (16/B); general widths: codes 2*pi and 2*pi + 1.  Returns the code
// indices of the low / high fp16 element and the operand's 2^s code scale.
template <int B>
__device__ inline void k_slot(int G, int nks, int ks, int p, int rk, bool& valid, int& j_lo, int& j_hi, int& s) {
  const int pi = G * nks * 4 + ks * 4 + p;
  valid = pi < rk / 2;
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    const int w = pi / PPW, u = pi % PPW;
    j_lo = w * (32 / B) + u;
    j_hi = j_lo + PPW;
    s = Pow2<B>::at(((ks * 4 + p) % PPW) * B);  // after the per-lane pre-shift of k_phase
  } else {
    j_lo = 2 * pi;
    j_hi = 2 * pi + 1;
    s = 0;
  }
}

// ----------------------------------------------------------------- per-tile phases
// Scores of one 64-token tile: four 16-token sub-tiles, C[head][token] on the
// matrix cores, written to S[token][GM] (log2 units before min/step are applied).
template <int B, int NKS, int GM>
__device__ __attribute__((always_inline)) inline void k_phase(rsrc_t rk_, uint32_t wkb, int t0, int tlast,
                                                              const u32x4 (&aq_hi)[4], const u32x4 (&aq_lo)[4],
                                                              float* S) {
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    constexpr int NWL = (NKS * 4 * B + 15) / 16;
    const int base = G * NKS * 4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      int tok = t0 + tt * 16 + n;
      tok = tok < tlast ? tok : tlast;
      uint32_t w[NWL];
      load_words<NWL>(rk_, (uint32_t)tok * wkb + 4u * (1 + base / PPW), w);
      if constexpr (NKS * 4 < PPW) w[0] >>= (base % PPW) * B;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 bop;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pl = ks * 4 + p;
          bop[p] = Pow2<B>::pair(w[pl / PPW], (pl % PPW) * B);
        }
        acc = mfma(aq_hi[ks], bop, acc);
        acc = mfma(aq_lo[ks], bop, acc);
      }
      if (4 * G < GM) *(f32x4*)(S + (tt * 16 + n) * GM + 4 * G) = acc;
    }
  } else {
    // general widths: one window load per pair, one sub-tile in flight
    constexpr uint32_t M = (1u << B) - 1u;
#pragma unroll 1
    for (int tt = 0; tt < 4; ++tt) {
      int tok = t0 + tt * 16 + n;
      tok = tok < tlast ? tok : tlast;
      const uint32_t rec = (uint32_t)tok * wkb;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 bop;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pi = G * NKS * 4 + ks * 4 + p;
          const uint32_t f = window(rk_, rec, 2 * pi * B);
          bop[p] = (f & M) | (((f >> B) & M) << 16);
        }
        acc = mfma(aq_hi[ks], bop, acc);
        acc = mfma(aq_lo[ks], bop, acc);
      }
      if (4 * G < GM) *(f32x4*)(S + (tt * 16 + n) * GM + 4 * G) = acc;
    }
  }
}

// One 32-token value step (tokens t0 .. t0+31): for each N-tile of 16 codes the
// B operand (lane n owns codes [n*NT, (n+1)*NT) of the 8 tokens of its lane
// group, one aligned field of NT*B bits for power-of-two widths) and its two
// MFMAs with A = p*step_V (hi, lo).
template <int B, int NT>
__device__ __attribute__((always_inline)) inline void v_phase(rsrc_t rv_, uint32_t wvb, int t0, int tlast,
                                                              u32x4 ahi, u32x4 alo, f32x4 (&acc2)[8]) {
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    constexpr int FS = NT * B;
    uint32_t f0[8], f1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int tok = t0 + 8 * G + e;
      tok = tok < tlast ? tok : tlast;
      const uint32_t rec = (uint32_t)tok * wvb + 4u;
      f1[e] = 0u;
      if constexpr (FS <= 16) {
        const int bit = n * FS;
        const uint32_t x = ld16(rv_, rec + 2u * (bit >> 4)) >> (bit & 15);
        f0[e] = FS == 16 ? x : (x & ((1u << FS) - 1u));
      } else if constexpr (FS == 32) {
        f0[e] = ld32(rv_, rec + 4u * n);
      } else {
        const u32x2 a = ld64(rv_, rec + 8u * n);
        f0[e] = a[0];
        f1[e] = a[1];
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int k = nt / PPW;  // 16-bit slice of the field
      u32x4 bop;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t fa = k < 2 ? f0[2 * p] : f1[2 * p];
        const uint32_t fb = k < 2 ? f0[2 * p + 1] : f1[2 * p + 1];
        const uint32_t y = (k & 1) ? ((fa >> 16) | (fb & 0xFFFF0000u)) : ((fa & 0xFFFFu) | (fb << 16));
        bop[p] = Pow2<B>::pair(y, (nt % PPW) * B);
      }
      acc2[nt] = mfma(ahi, bop, acc2[nt]);
      acc2[nt] = mfma(alo, bop, acc2[nt]);
    }
  } else {
    constexpr uint32_t M = (1u << B) - 1u;
    const int fbit = n * NT * B;  // first bit of the lane's NT codes
    uint32_t w0[8], w1[8], w2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int tok = t0 + 8 * G + e;
      tok = tok < tlast ? tok : tlast;
      const uint32_t off = (uint32_t)tok * wvb + 4u * (1 + (fbit >> 5));
      const u32x2 a = ld64(rv_, off);
      w0[e] = a[0];
      w1[e] = a[1];
      w2[e] = ld32(rv_, off + 8u);
    }
    const int o0 = fbit & 31;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int o = o0 + nt * B;  // < 32 + 56
      u32x4 bop;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t ca = (o < 32 ? __builtin_amdgcn_alignbit(w1[2 * p], w0[2 * p], o)
                                    : __builtin_amdgcn_alignbit(w2[2 * p], w1[2 * p], o - 32)) & M;
        const uint32_t cb = (o < 32 ? __builtin_amdgcn_alignbit(w1[2 * p + 1], w0[2 * p + 1], o)
                                    : __builtin_amdgcn_alignbit(w2[2 * p + 1], w1[2 * p + 1], o - 32)) & M;
        bop[p] = ca | (cb << 16);
      }
      acc2[nt] = mfma(ahi, bop, acc2[nt]);
      acc2[nt] = mfma(alo, bop, acc2[nt]);
    }
  }
}

// Key operand (A of the score MFMA): row = head (lane % 16), element of pair slot
// = q~_j * 2^(E_head - s), split into fp16 hi + lo.
template <int B>
__device__ inline void build_aq(const float* qt, const float* sc, int g, int rk, u32x4 (&aq_hi)[4],
                                u32x4 (&aq_lo)[4]) {
  const int lane = threadIdx.x & 63, i = lane & 15, G = lane >> 4;
  const int nks = rk >= 32 ? rk / 32 : 1;
  const int E = i < g ? (int)sc[2 * kMaxGroup + i] : 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      bool valid;
      int jl, jh, sh;
      k_slot<B>(G, nks, ks, p, rk, valid, jl, jh, sh);
      float xl = 0.0f, xh = 0.0f;
      if (valid && i < g && ks < nks) {
        xl = ldexpf(qt[i * kMaxRank + jl], E - sh);
        xh = ldexpf(qt[i * kMaxRank + jh], E - sh);
      }
      const _Float16 hl = (_Float16)xl, hh = (_Float16)xh;
      const _Float16 ll = (_Float16)(xl - (float)hl), lh = (_Float16)(xh - (float)hh);
      aq_hi[ks][p] = h2u(hl) | (h2u(hh) << 16);
      aq_lo[ks][p] = h2u(ll) | (h2u(lh) << 16);
    }
  }
}

// 2^s code scale of value N-tile nt (power-of-two widths; general widths use s = 0).
__device__ inline int v_shift(int B, int nt) {
  switch (B) {
    case 2: return Pow2<2>::at((nt % Pow2<2>::kPerHalf) * 2);
    case 4: return Pow2<4>::at((nt % Pow2<4>::kPerHalf) * 4);
    case 8: return Pow2<8>::at((nt % Pow2<8>::kPerHalf) * 8);
    default: return 0;
  }
}

#define KVTC_K_CASE(B)                                                              \
  case B:                                                                           \
    if (nks == 1) k_phase<B, 1, GM>(rk_, wkb, t0, tlast, aq_hi, aq_lo, S);          \
    else if (nks == 2) k_phase<B, 2, GM>(rk_, wkb, t0, tlast, aq_hi, aq_lo, S);     \
    else k_phase<B, 4, GM>(rk_, wkb, t0, tlast, aq_hi, aq_lo, S);                   \
    break;
#define KVTC_V_CASE(B)                                                              \
  case B:                                                                           \
    if (NT == 1) v_phase<B, 1>(rv_, wvb, t0 + 32 * kk, tlast, ahi, alo, acc2);       \
    else if (NT == 2) v_phase<B, 2>(rv_, wvb, t0 + 32 * kk, tlast, ahi, alo, acc2);  \
    else if (NT == 4) v_phase<B, 4>(rv_, wvb, t0 + 32 * kk, tlast, ahi, alo, acc2);  \
    else v_phase<B, 8>(rv_, wvb, t0 + 32 * kk, tlast, ahi, alo, acc2);               \
    break;

// ----------------------------------------------------------------- kernel
// Grid (n_wg, n_kv_heads, batch), 256 threads; GM bounds the GQA group (g <= GM).
// Workgroup x covers tokens [x*split_tokens, (x+1)*split_tokens), a quarter per
// wave; each wave runs its own online softmax and the four states are merged in
// LDS into one partial (m, l, o~[r_V]) per query head and split.
template <int GM, bool GEN>
__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a) {
  extern __shared__ float lds[];
  constexpr int WA = 128 * GM;  // words per wave area
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the token loop scalar
  const HeadDesc& hd = a.heads.h[h];
  // head parameters are wave-uniform; readfirstlane keeps them (and every branch on them) scalar
  const int g = __builtin_amdgcn_readfirstlane(a.group), rk = __builtin_amdgcn_readfirstlane(hd.rk);
  const int rv = __builtin_amdgcn_readfirstlane(hd.rv);
  const int bk = __builtin_amdgcn_readfirstlane(hd.bk), bv = __builtin_amdgcn_readfirstlane(hd.bv);
  const int nks = rk >= 32 ? rk / 32 : 1;
  const int NT = rv / 16;
  const int64_t bq0 = (int64_t)b * a.n_q_heads + (int64_t)h * g;

  float* sc = lds;                        // sq[16] | 2^(24-E)[16] | E[16] | pad
  float* ml = lds + 64;                   // per wave: m[16] l[16] c[16]
  float* areas = lds + 64 + kWaves * 48;  // per wave: WA words
  float* wl = areas + wave * WA;

  // ---- prologue: q~ = scale * log2(e) * P_K^T q of the g heads (raw q and q~ over the wave areas)
  float* q_raw = areas;
  float* qt = areas + GM * kHeadDim;
  for (int i = tid; i < g * kHeadDim; i += 256) {
    const int64_t off = (bq0 + i / kHeadDim) * kHeadDim + (i % kHeadDim);
    q_raw[i] = a.dtype == 0 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off];
  }
  __syncthreads();
  {
    const float* PK = a.basis_k + hd.boff_k;
    for (int o = tid; o < g * rk; o += 256) {
      const int hh = o / rk, j = o % rk;
      const float* qh = q_raw + hh * kHeadDim;
      float acc = 0.0f;
#pragma unroll 8
      for (int i = 0; i < kHeadDim; ++i) acc = fmaf(PK[i * rk + j], qh[i], acc);
      qt[hh * kMaxRank + j] = acc * a.scale_log2;
    }
  }
  __syncthreads();
  if (tid < g) {
    float sum = 0.0f, mx = 0.0f;
    for (int j = 0; j < rk; ++j) {
      const float v = qt[tid * kMaxRank + j];
      sum += v;
      mx = fmaxf(mx, fabsf(v));
    }
    int e = 0;
    if (mx > 0.0f) {
      frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
      e = 14 - e;      // max |q~| * 2^E < 2^14
    }
    sc[tid] = sum;
    sc[kMaxGroup + tid] = ldexpf(1.0f, 24 - e);
    sc[2 * kMaxGroup + tid] = (float)e;
  }
  __syncthreads();
  u32x4 aq_hi[4], aq_lo[4];
  if (pow2_bits(bk)) {
    switch (bk) {
      case 2: build_aq<2>(qt, sc, g, rk, aq_hi, aq_lo); break;
      case 4: build_aq<4>(qt, sc, g, rk, aq_hi, aq_lo); break;
      default: build_aq<8>(qt, sc, g, rk, aq_hi, aq_lo); break;
    }
  } else {
    build_aq<3>(qt, sc, g, rk, aq_hi, aq_lo);  // general widths share the adjacent-pair slot map
  }
  float sq[GM], kf[GM];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    sq[hh] = uniform(sc[hh]);
    kf[hh] = uniform(sc[kMaxGroup + hh]);
  }
  __syncthreads();  // q~ in the wave areas is no longer needed
  float* S = wl;                               // [64][GM] fp32
  _Float16* P = (_Float16*)(wl + 64 * GM);     // [2][GM][64] fp16, rows >= g stay zero
  for (int i = lane; i < GM * 64; i += 64) ((uint32_t*)P)[i] = 0u;

  // ---- this wave's token range and cache regions
  const int wq = (int)(a.split_tokens / kWaves);
  const int t_begin = (int)blockIdx.x * (int)a.split_tokens + wave * wq;
  int t_end = t_begin + wq;
  if (t_end > (int)a.n_tokens) t_end = (int)a.n_tokens;
  const uint32_t wkb = 4u * hd.wk, wvb = 4u * hd.wv;
  const uint32_t* kreg = a.cache_k + hd.base_k + (int64_t)b * a.capacity * hd.wk;
  const uint32_t* vreg = a.cache_v + hd.base_v + (int64_t)b * a.capacity * hd.wv;
  const rsrc_t rk_ = make_rsrc(kreg, (uint32_t)a.capacity * wkb);
  const rsrc_t rv_ = make_rsrc(vreg, (uint32_t)a.capacity * wvb);

  float m_run[GM], l_run[GM], c_run[GM];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.0f;
    c_run[hh] = 0.0f;
  }
  f32x4 acc2[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc2[nt] = {0.f, 0.f, 0.f, 0.f};
  lds_fence();

  for (int t0 = t_begin; t0 < t_end; t0 += kTileT) {
    const int tlast = t_end - 1;
    if constexpr (GEN) {
      switch (bk) {
        KVTC_K_CASE(2) KVTC_K_CASE(3) KVTC_K_CASE(4) KVTC_K_CASE(5) KVTC_K_CASE(6) KVTC_K_CASE(7) KVTC_K_CASE(8)
      }
    } else {
      switch (bk) { KVTC_K_CASE(2) KVTC_K_CASE(4) KVTC_K_CASE(8) }
    }
    // ---- online softmax, one token per lane
    const int tok = t0 + lane;
    const bool valid = tok < t_end;
    const uint32_t tokc = (uint32_t)(valid ? tok : tlast);
    const uint32_t kh = ld32(rk_, tokc * wkb);
    const uint32_t vh = ld32(rv_, tokc * wvb);
    const float muk = f16_bits_to_f32(kh & 0xFFFFu), sgk = f16_bits_to_f32(kh >> 16);
    const float muv = f16_bits_to_f32(vh & 0xFFFFu), sgv = f16_bits_to_f32(vh >> 16);
    lds_fence();
    float s[GM];
#pragma unroll
    for (int q4 = 0; q4 < GM / 4; ++q4) {
      const f32x4 d = *(const f32x4*)(S + lane * GM + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hh = 4 * q4 + e;
        s[hh] = (valid && hh < g) ? fmaf(sgk * kf[hh], d[e], muk * sq[hh]) : -__builtin_inff();
      }
    }
    // lazy maximum: the reference only moves when a score exceeds it, so p <= 1
    bool up = false;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) up |= s[hh] > m_run[hh];
    if (__any(up)) {
      float alpha[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        alpha[hh] = 1.0f;
        if (hh < g) {
          const float mn = uniform(fmaxf(m_run[hh], wave_max(s[hh])));
          if (mn > m_run[hh]) {
            alpha[hh] = exp2f(m_run[hh] - mn);  // 0 while the old reference is -inf
            m_run[hh] = mn;
          }
          l_run[hh] *= alpha[hh];
          c_run[hh] *= alpha[hh];
        }
      }
      // value accumulators: lane (n, G) holds heads 4G..4G+3
      lds_fence();
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) S[hh] = alpha[hh];
      }
      lds_fence();
      const int G = lane >> 4;
      if (4 * G < GM) {
        const f32x4 f = *(const f32x4*)(S + 4 * G);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc2[nt] *= f;
      }
    }
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh < g) {
        const float p = exp2f(s[hh] - m_run[hh]);
        l_run[hh] += p;
        c_run[hh] = fmaf(p, muv, c_run[hh]);
        const float x = p * sgv;
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        P[hh * 64 + lane] = hi;
        P[GM * 64 + hh * 64 + lane] = lo;
      }
    }
    lds_fence();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int n = lane & 15, G = lane >> 4;
      u32x4 ahi = {0u, 0u, 0u, 0u}, alo = {0u, 0u, 0u, 0u};
      if (n < GM) {
        ahi = *(const u32x4*)(P + n * 64 + 32 * kk + 8 * G);
        alo = *(const u32x4*)(P + GM * 64 + n * 64 + 32 * kk + 8 * G);
      }
      if constexpr (GEN) {
        switch (bv) {
          KVTC_V_CASE(2) KVTC_V_CASE(3) KVTC_V_CASE(4) KVTC_V_CASE(5) KVTC_V_CASE(6) KVTC_V_CASE(7) KVTC_V_CASE(8)
        }
      } else {
        switch (bv) { KVTC_V_CASE(2) KVTC_V_CASE(4) KVTC_V_CASE(8) }
      }
    }
    lds_fence();
  }

  // ---- wave partial: m, l, sum of p*min (per head), o~[head][j] in natural code order
  float* mlw = ml + wave * 48;
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const float ls = wave_sum(l_run[hh]);
    const float cs = wave_sum(c_run[hh]);
    if (lane == 0 && hh < g) {
      mlw[hh] = m_run[hh];
      mlw[16 + hh] = ls;
      mlw[32 + hh] = cs;
    }
  }
  lds_fence();
  {
    const int n = lane & 15, G = lane >> 4;
    if (4 * G < GM) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        if (nt < NT) {
          const float f = ldexpf(1.0f, 24 - v_shift(bv, nt));
          const int j = n * NT + nt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int hh = 4 * G + e;
            if (hh < g) wl[hh * rv + j] = fmaf(acc2[nt][e], f, mlw[32 + hh]);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- merge the four wave partials, one partial per query head
  float* part0 = a.part + (bq0 * a.n_splits + blockIdx.x) * (int64_t)kPartStride;
  for (int o = tid; o < g * rv; o += 256) {
    const int hh = o / rv, j = o % rv;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if ((int)blockIdx.x * (int)a.split_tokens + w * wq < (int)a.n_tokens) M = fmaxf(M, ml[w * 48 + hh]);
    const float mu = M == -__builtin_inff() ? 0.0f : M;
    float acc = 0.0f, lacc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if ((int)blockIdx.x * (int)a.split_tokens + w * wq < (int)a.n_tokens) {
        const float wgt = exp2f(ml[w * 48 + hh] - mu);
        acc = fmaf(wgt, areas[w * WA + hh * rv + j], acc);
        lacc = fmaf(wgt, ml[w * 48 + 16 + hh], lacc);
      }
    }
    float* ph = part0 + (int64_t)hh * a.n_splits * kPartStride;
    ph[2 + j] = acc;
    if (j == 0) {
      ph[0] = M;
      ph[1] = lacc;
    }
  }
}

// ----------------------------------------------------------------- combine + back-projection
// Grid batch * n_q_heads, 256 threads.  Log-sum-exp merge of the split partials,
// then o = P_V o~ / l (d x r_V back-projection of the value sum).
__global__ __launch_bounds__(256) void combine_kernel(AttendArgs a) {
  __shared__ float wgt[1024];
  __shared__ float ot[4][kMaxRank];
  __shared__ float red[8];
  const int bq = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.n_tokens <= 0) {  // attention over no tokens is defined as zero output
    if (tid < kHeadDim) a.out[(int64_t)bq * kHeadDim + tid] = 0.0f;
    return;
  }
  const int hq = bq % a.n_q_heads;
  const HeadDesc& hd = a.heads.h[hq / a.group];
  const int rv = hd.rv, ns = a.n_splits;
  const float* part = a.part + (int64_t)bq * ns * kPartStride;
  float M = -__builtin_inff();
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, part[(int64_t)s * kPartStride]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mu = M == -__builtin_inff() ? 0.0f : M;
  float L = 0.0f;
  for (int s = tid; s < ns; s += 256) {
    const float* ps = part + (int64_t)s * kPartStride;
    const float w = exp2f(ps[0] - mu);
    if (s < 1024) wgt[s] = w;
    L = fmaf(w, ps[1], L);
  }
  L = wave_sum(L);
  if (lane == 0) red[4 + wave] = L;
  __syncthreads();
  L = red[4] + red[5] + red[6] + red[7];
  // o~: wave w sums splits w, w+4, ...; lanes cover the code indices
  for (int j = lane; j < rv; j += 64) {
    float acc0 = 0.0f, acc1 = 0.0f;
    int s = wave;
    for (; s + 4 < ns; s += 8) {
      const float w0 = s < 1024 ? wgt[s] : exp2f(part[(int64_t)s * kPartStride] - mu);
      const float w1 = s + 4 < 1024 ? wgt[s + 4] : exp2f(part[(int64_t)(s + 4) * kPartStride] - mu);
      acc0 = fmaf(w0, part[(int64_t)s * kPartStride + 2 + j], acc0);
      acc1 = fmaf(w1, part[(int64_t)(s + 4) * kPartStride + 2 + j], acc1);
    }
    for (; s < ns; s += 4) {
      const float w0 = s < 1024 ? wgt[s] : exp2f(part[(int64_t)s * kPartStride] - mu);
      acc0 = fmaf(w0, part[(int64_t)s * kPartStride + 2 + j], acc0);
    }
    ot[wave][j] = acc0 + acc1;
  }
  __syncthreads();
  if (tid < rv) ot[0][tid] = ot[0][tid] + ot[1][tid] + ot[2][tid] + ot[3][tid];
  __syncthreads();
  // back-projection: wave w covers rows i = 32w .. 32w+31, two lanes per row
  const float* PV = a.basis_v + hd.boff_v;
  const int i = wave * 32 + (lane >> 1), half = lane & 1;
  float acc = 0.0f;
  for (int j = half; j < rv; j += 2) acc = fmaf(PV[(int64_t)i * rv + j], ot[0][j], acc);
  acc += __shfl_xor(acc, 1);
  if (half == 0) a.out[(int64_t)bq * kHeadDim + i] = L > 0.0f ? acc / L : 0.0f;
}

template <int GM, bool GEN>
static hipError_t launch_gm(const AttendArgs& a, hipStream_t s) {
  const size_t lds = (64 + kWaves * 48 + kWaves * 128 * GM) * sizeof(float);
  const dim3 grid((unsigned)a.n_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attend_mfma_kernel<GM, GEN>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <bool GEN>
static hipError_t launch_widths(const AttendArgs& a, hipStream_t s) {
  return a.group <= 4 ? launch_gm<4, GEN>(a, s) : a.group <= 8 ? launch_gm<8, GEN>(a, s) : launch_gm<16, GEN>(a, s);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.n_tokens > 0) {
    // layouts whose widths are all powers of two use the instance without the general-width paths
    bool gen = false;
    for (int h = 0; h < a.n_kv_heads; ++h) {
      const HeadDesc& d = a.heads.h[h];
      gen |= !(pow2_bits(d.bk) && pow2_bits(d.bv));
    }
    const hipError_t e = gen ? launch_widths<true>(a, s) : launch_widths<false>(a, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(a.batch * a.n_q_heads)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvtc
