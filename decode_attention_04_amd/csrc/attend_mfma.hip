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

// Wave-uniform maximum with DPP row operations (pairs, quads, half rows, rows),
// then the four row results through scalar reads.
template <int CTRL>
__device__ inline float dpp_max(float x) {
  const int y = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
  return fmaxf(x, __builtin_bit_cast(float, y));
}
__device__ inline float wave_max_uniform(float x) {
  x = dpp_max<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x141>(x);  // row_half_mirror
  x = dpp_max<0x140>(x);  // row_mirror
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}


__device__ inline float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ----------------------------------------------------------------- record tiles in LDS
// One buffer resource per (sequence, KV head) cache region: 32-bit byte offsets,
// loads past the region return zero.  Tiles of 64 consecutive records are copied
// HBM -> LDS with buffer_load_dwordx4 ... lds (16 bytes per lane, lane-contiguous
// in LDS), so the copy of the next tile is in flight while the current one is
// unpacked, and every unpacking access is an LDS read.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copy `nbytes` starting at byte `src` of the region to LDS `dst` in 16-byte
// chunks (up to 12 bytes past the end are copied too).
__device__ inline void tile_copy(rsrc_t r, uint32_t src, uint32_t nbytes, uint32_t* dst) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t n16 = (nbytes + 15u) >> 4;
  uint32_t c = 0;
  for (; c + 64 <= n16; c += 64)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 4 * c), 16, (int)(src + 16u * (c + lane)), 0, 0, 0);
  if (c + lane < n16)  // tail: only the lanes whose 16 bytes belong to the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 4 * c), 16, (int)(src + 16u * (c + lane)), 0, 0, 0);
}

__device__ inline void wait_tiles() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N>
__device__ inline void lds_words(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N == 1) {
    w[0] = p[0];
  } else if constexpr (N == 2) {
    const u32x2a a = *(const u32x2a*)p;
    w[0] = a[0]; w[1] = a[1];
  } else {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      const u32x4a a = *(const u32x4a*)(p + k);
      w[k] = a[0]; w[k + 1] = a[1]; w[k + 2] = a[2]; w[k + 3] = a[3];
    }
  }
}

// B adjacent-code bits starting at stream bit `bit` of a record in LDS (low code in bits 0..).
__device__ inline uint32_t lds_window(const uint32_t* rec, int bit) {
  const uint32_t* p = rec + 1 + (bit >> 5);
  return __builtin_amdgcn_alignbit(p[1], p[0], bit & 31);
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

// ----------------------------------------------------------------- per-tile phases (records in LDS)
// Scores of one 64-token tile: four 16-token sub-tiles, C[head][token] on the
// matrix cores, written to S[token][GM] (log2 units before min/step are applied).
// kt: the tile's records (wk words each); tokens past `nlast` read record nlast.
template <int B, int NKS, int GM>
__device__ __attribute__((always_inline)) inline void k_phase(const uint32_t* kt, int wk,
                                                              const u32x4 (&aq_hi)[4], const u32x4 (&aq_lo)[4],
                                                              float* S) {
  // tokens past the tile's last record read stale LDS: their codes are finite and
  // their scores are replaced by -inf before the softmax
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  const uint32_t* rec0 = kt + n * wk;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const uint32_t* rec = rec0 + tt * 16 * wk;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (pow2_bits(B)) {
      constexpr int PPW = Pow2<B>::kPerHalf;
      constexpr int NWL = (NKS * 4 * B + 15) / 16;
      const int base = G * NKS * 4;
      uint32_t w[NWL];
      lds_words<NWL>(rec + 1 + base / PPW, w);
      if constexpr (NKS * 4 < PPW) w[0] >>= (base % PPW) * B;
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
    } else {
      constexpr uint32_t M = (1u << B) - 1u;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 bop;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pi = G * NKS * 4 + ks * 4 + p;
          const uint32_t f = lds_window(rec, 2 * pi * B);
          bop[p] = (f & M) | (((f >> B) & M) << 16);
        }
        acc = mfma(aq_hi[ks], bop, acc);
        acc = mfma(aq_lo[ks], bop, acc);
      }
    }
    // S[token][GM]; lanes holding head rows >= GM (all zero) store into the dump slot
    *(f32x4*)(S + (4 * G < GM ? (tt * 16 + n) * GM + 4 * G : 64 * GM)) = acc;
  }
}

// One 32-token value step (tile tokens 32*kk .. 32*kk+31): for each N-tile of 16
// codes the B operand (lane n owns codes [n*NT, (n+1)*NT) of the 8 tokens of its
// lane group, one aligned field of NT*B bits for power-of-two widths) and its two
// MFMAs with A = p*step_V (hi, lo).
template <int B, int NT>
__device__ __attribute__((always_inline)) inline void v_phase(const uint32_t* vt, int wv, int kk,
                                                              u32x4 ahi, u32x4 alo, f32x4 (&acc2)[8]) {
  // tokens past the tile's last record carry p = 0 in A, so their (finite) codes add nothing
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  const uint32_t* rec0 = vt + (32 * kk + 8 * G) * wv + 1;
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    constexpr int FS = NT * B;
    uint32_t f0[8], f1[8];
    const int bit = n * FS;
    const uint16_t* h0 = (const uint16_t*)rec0 + (bit >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f1[e] = 0u;
      if constexpr (FS <= 16) {
        const uint32_t x = (uint32_t)h0[2 * e * wv] >> (bit & 15);
        f0[e] = FS == 16 ? x : (x & ((1u << FS) - 1u));
      } else if constexpr (FS == 32) {
        f0[e] = rec0[e * wv + n];
      } else {
        const u32x2a a = *(const u32x2a*)(rec0 + e * wv + 2 * n);
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
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int bit = (n * NT + nt) * B;
      u32x4 bop;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t ca = lds_window(rec0 - 1 + (2 * p) * wv, bit) & M;
        const uint32_t cb = lds_window(rec0 - 1 + (2 * p + 1) * wv, bit) & M;
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
    if (nks == 1) k_phase<B, 1, GM>(kt, wk, aq_hi, aq_lo, S);                            \
    else if (nks == 2) k_phase<B, 2, GM>(kt, wk, aq_hi, aq_lo, S);                       \
    else k_phase<B, 4, GM>(kt, wk, aq_hi, aq_lo, S);                                     \
    break;
#define KVTC_V_CASE(B)                                                              \
  case B:                                                                           \
    if (NT == 1) v_phase<B, 1>(vt, wv, kk, ahi, alo, acc2);                          \
    else if (NT == 2) v_phase<B, 2>(vt, wv, kk, ahi, alo, acc2);                     \
    else if (NT == 4) v_phase<B, 4>(vt, wv, kk, ahi, alo, acc2);                     \
    else v_phase<B, 8>(vt, wv, kk, ahi, alo, acc2);                                  \
    break;

// Words of LDS per wave: tile buffers for K and V (nbuf each), the scores
// S[64][GM] plus a 4-word dump slot for the score rows >= GM, and the
// probabilities P[2][GM][64] (fp16) plus a 4-word zero slot read as rows >= GM.
__host__ __device__ constexpr int score_words(int gm) { return 64 * gm + 4 + gm * 64 + 4; }
__host__ __device__ inline int wave_lds_words(int kbuf_words, int vbuf_words, int nbuf, int gm) {
  return nbuf * (kbuf_words + vbuf_words) + score_words(gm);
}

// ----------------------------------------------------------------- kernel
// Grid (n_wg, n_kv_heads, batch), 256 threads; GM bounds the GQA group (g <= GM);
// GEN adds the general-width (3, 5, 6, 7 bits) unpacking paths.  Workgroup x
// covers tokens [x*split_tokens, (x+1)*split_tokens), a quarter per wave; each
// wave streams its records through LDS in 64-token tiles and runs its own online
// softmax; the four wave states are merged in LDS into one partial (m, l, o~[r_V])
// per query head and split.
template <int GM, bool GEN>
__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a) {
  extern __shared__ float lds[];
  const int WA = wave_lds_words(a.kbuf_words, a.vbuf_words, a.nbuf, GM);
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

  // ---- this wave's token range and cache regions; start streaming the first tile
  const int wq = (int)(a.split_tokens / kWaves);
  const int t_begin = (int)blockIdx.x * (int)a.split_tokens + wave * wq;
  int t_end = t_begin + wq;
  if (t_end > (int)a.n_tokens) t_end = (int)a.n_tokens;
  const int wk = hd.wk, wv = hd.wv;
  const uint32_t* kreg = a.cache_k + hd.base_k + (int64_t)b * a.capacity * wk;
  const uint32_t* vreg = a.cache_v + hd.base_v + (int64_t)b * a.capacity * wv;
  const rsrc_t rk_ = make_rsrc(kreg, (uint32_t)a.capacity * 4u * wk);
  const rsrc_t rv_ = make_rsrc(vreg, (uint32_t)a.capacity * 4u * wv);
  uint32_t* ktile = (uint32_t*)wl;                          // [nbuf][kbuf_words]
  uint32_t* vtile = ktile + a.nbuf * a.kbuf_words;          // [nbuf][vbuf_words]
  float* S = (float*)(vtile + a.nbuf * a.vbuf_words);       // [64][GM] fp32, then a dump slot
  _Float16* P = (_Float16*)(S + 64 * GM + 4);               // [2][GM][64] fp16 (rows >= g stay zero), zero slot

  // ---- prologue: q~ = scale * log2(e) * P_K^T q of the g heads (raw q and q~ in the
  // score areas of waves 0..3, which are not in use yet)
  // q (g x 128) and q~ (g x 128) over the tile buffers of waves 2 and 3, which start
  // streaming only after the prologue
  float* q_raw = areas + 2 * WA;
  float* qt = areas + 3 * WA;
  for (int i = tid; i < g * kHeadDim; i += 256) {
    const int64_t off = (bq0 + i / kHeadDim) * kHeadDim + (i % kHeadDim);
    q_raw[i] = a.dtype == 0 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off];
  }
  const int n0 = (t_end - t_begin) < kTileT ? (t_end - t_begin) : kTileT;
  if (wave < 2 && t_begin < t_end) {  // waves 2 and 3 lend their buffers to the prologue
    tile_copy(rk_, (uint32_t)t_begin * 4u * wk, (uint32_t)n0 * 4u * wk, ktile);
    tile_copy(rv_, (uint32_t)t_begin * 4u * wv, (uint32_t)n0 * 4u * wv, vtile);
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
  __syncthreads();  // the prologue's q and q~ are consumed
  if (wave >= 2 && t_begin < t_end) {
    tile_copy(rk_, (uint32_t)t_begin * 4u * wk, (uint32_t)n0 * 4u * wk, ktile);
    tile_copy(rv_, (uint32_t)t_begin * 4u * wv, (uint32_t)n0 * 4u * wv, vtile);
  }
  for (int i = lane; i < GM * 64 + 4; i += 64) ((uint32_t*)P)[i] = 0u;

  // running state: reference maximum (finite start, so heads >= g never form -inf - -inf),
  // per-lane partial sums of p and p * min_V, value accumulators of 8 N-tiles
  float m_run[GM], l_run[GM], c_run[GM];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m_run[hh] = -1e30f;
    l_run[hh] = 0.0f;
    c_run[hh] = 0.0f;
  }
  f32x4 acc2[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc2[nt] = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, G = lane >> 4;
  const int hoff_k = lane * wk, hoff_v = lane * wv;  // this lane's token header in a tile
  const uint32_t* kt = ktile;
  const uint32_t* vt = vtile;
  uint32_t* kt_next = ktile + (a.nbuf == 2 ? a.kbuf_words : 0);
  uint32_t* vt_next = vtile + (a.nbuf == 2 ? a.vbuf_words : 0);
  lds_fence();

  for (int t0 = t_begin; t0 < t_end; t0 += kTileT) {
    const int nvalid = t_end - t0 < kTileT ? t_end - t0 : kTileT;
    wait_tiles();  // this tile is in LDS
    const int t1 = t0 + kTileT;
    if (a.nbuf == 2 && t1 < t_end) {  // next tile streams in while this one is processed
      const int n1 = (t_end - t1) < kTileT ? (t_end - t1) : kTileT;
      tile_copy(rk_, (uint32_t)t1 * 4u * wk, (uint32_t)n1 * 4u * wk, kt_next);
      tile_copy(rv_, (uint32_t)t1 * 4u * wv, (uint32_t)n1 * 4u * wv, vt_next);
    }
    if constexpr (GEN) {
      switch (bk) {
        KVTC_K_CASE(2) KVTC_K_CASE(3) KVTC_K_CASE(4) KVTC_K_CASE(5) KVTC_K_CASE(6) KVTC_K_CASE(7) KVTC_K_CASE(8)
      }
    } else {
      switch (bk) { KVTC_K_CASE(2) KVTC_K_CASE(4) KVTC_K_CASE(8) }
    }
    // ---- online softmax, one token per lane (branch-free over heads)
    const bool valid = lane < nvalid;
    const uint32_t kh = kt[hoff_k];
    const uint32_t vh = vt[hoff_v];
    const float muk = f16_bits_to_f32(kh & 0xFFFFu), sgk = f16_bits_to_f32(kh >> 16);
    const float muv = valid ? f16_bits_to_f32(vh & 0xFFFFu) : 0.0f;
    const float sgv = valid ? f16_bits_to_f32(vh >> 16) : 0.0f;
    lds_fence();
    float s[GM];
#pragma unroll
    for (int q4 = 0; q4 < GM / 4; ++q4) {
      const f32x4 d = *(const f32x4*)(S + lane * GM + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hh = 4 * q4 + e;
        const float x = fmaf(sgk * kf[hh], d[e], muk * sq[hh]);
        s[hh] = (valid && hh < g) ? x : -__builtin_inff();
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
        const float mn = fmaxf(m_run[hh], wave_max_uniform(s[hh]));
        alpha[hh] = exp2f(m_run[hh] - mn);  // 1 if unchanged, 0 on the first tile
        m_run[hh] = mn;
        l_run[hh] *= alpha[hh];
        c_run[hh] *= alpha[hh];
      }
      // value accumulators: lane (n, G) holds heads 4G..4G+3
      lds_fence();
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) S[hh] = alpha[hh];
      }
      lds_fence();
      const f32x4 f = 4 * G < GM ? *(const f32x4*)(S + 4 * G) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc2[nt] *= f;
    }
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      const float p = exp2f(s[hh] - m_run[hh]);
      l_run[hh] += p;
      c_run[hh] = fmaf(p, muv, c_run[hh]);
      const float x = p * sgv;
      const _Float16 hi = (_Float16)x;
      const _Float16 lo = (_Float16)(x - (float)hi);
      P[hh * 64 + lane] = hi;
      P[GM * 64 + hh * 64 + lane] = lo;
    }
    lds_fence();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // A rows >= GM read the zero slot
      const u32x4 ahi = *(const u32x4*)(P + (n < GM ? n * 64 + 32 * kk + 8 * G : 2 * GM * 64));
      const u32x4 alo = *(const u32x4*)(P + (n < GM ? GM * 64 + n * 64 + 32 * kk + 8 * G : 2 * GM * 64));
      if constexpr (GEN) {
        switch (bv) {
          KVTC_V_CASE(2) KVTC_V_CASE(3) KVTC_V_CASE(4) KVTC_V_CASE(5) KVTC_V_CASE(6) KVTC_V_CASE(7) KVTC_V_CASE(8)
        }
      } else {
        switch (bv) { KVTC_V_CASE(2) KVTC_V_CASE(4) KVTC_V_CASE(8) }
      }
    }
    lds_fence();
    if (a.nbuf == 1) {
      if (t1 < t_end) {  // single buffer: refill after the tile is consumed
        const int n1 = (t_end - t1) < kTileT ? (t_end - t1) : kTileT;
        tile_copy(rk_, (uint32_t)t1 * 4u * wk, (uint32_t)n1 * 4u * wk, ktile);
        tile_copy(rv_, (uint32_t)t1 * 4u * wv, (uint32_t)n1 * 4u * wv, vtile);
      }
    } else {
      const uint32_t* tk = kt;
      kt = kt_next;
      kt_next = (uint32_t*)tk;
      const uint32_t* tv = vt;
      vt = vt_next;
      vt_next = (uint32_t*)tv;
    }
  }
  wait_tiles();

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
// Grid (n_kv_heads, batch), 256 threads: the g query heads of one KV head.  Each
// wave merges the split partials of its heads with a running log-sum-exp (one
// pass, loads independent across splits); then o = P_V o~ / l with P_V read once
// for all g heads (thread pair per output row, half the codes each).
__global__ __launch_bounds__(256) void combine_kernel(AttendArgs a) {
  __shared__ float ot[kMaxGroup][kMaxRank];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = a.group;
  const int64_t bq0 = (int64_t)b * a.n_q_heads + (int64_t)h * g;
  if (a.n_tokens <= 0) {  // attention over no tokens is defined as zero output
    for (int i = tid; i < g * kHeadDim; i += 256) a.out[bq0 * kHeadDim + i] = 0.0f;
    return;
  }
  const HeadDesc& hd = a.heads.h[h];
  const int rv = hd.rv, ns = a.n_splits;
  for (int hh = wave; hh < g; hh += kWaves) {
    const float* part = a.part + (bq0 + hh) * ns * (int64_t)kPartStride;
    float M = -__builtin_inff(), L = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const float* ps = part + (int64_t)s * kPartStride;
      const float m = ps[0], l = ps[1];
      const float o0 = lane < rv ? ps[2 + lane] : 0.0f;
      const float o1 = lane + 64 < rv ? ps[2 + 64 + lane] : 0.0f;
      const float mn = fmaxf(M, m);
      const float mu = mn == -__builtin_inff() ? 0.0f : mn;
      const float sc = exp2f(M - mu), w = exp2f(m - mu);
      L = fmaf(L, sc, w * l);
      a0 = fmaf(a0, sc, w * o0);
      a1 = fmaf(a1, sc, w * o1);
      M = mn;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (lane < rv) ot[hh][lane] = a0 * inv;
    if (lane + 64 < rv) ot[hh][lane + 64] = a1 * inv;
  }
  __syncthreads();
  const float* PV = a.basis_v + hd.boff_v;
  const int i = tid >> 1, half = tid & 1;
  const int jh = rv / 2;
  float acc[kMaxGroup];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) acc[hh] = 0.0f;
  const float* row = PV + (int64_t)i * rv + half * jh;
  for (int j = 0; j < jh; j += 4) {
    const float4 pv = *(const float4*)(row + j);
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      if (hh < g) {
        const float* o = &ot[hh][half * jh + j];
        acc[hh] = fmaf(pv.x, o[0], fmaf(pv.y, o[1], fmaf(pv.z, o[2], fmaf(pv.w, o[3], acc[hh]))));
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    if (hh < g) {
      const float v = acc[hh] + __shfl_xor(acc[hh], 1);
      if (half == 0) a.out[(bq0 + hh) * kHeadDim + i] = v;
    }
  }
}

template <int GM, bool GEN>
static hipError_t launch_gm(const AttendArgs& a, hipStream_t s) {
  const size_t lds = (64 + kWaves * 48 + kWaves * (size_t)wave_lds_words(a.kbuf_words, a.vbuf_words, a.nbuf, GM)) *
                     sizeof(float);
  const dim3 grid((unsigned)a.n_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch);
  hipLaunchKernelGGL((attend_mfma_kernel<GM, GEN>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <bool GEN>
static hipError_t launch_widths(const AttendArgs& a, hipStream_t s) {
  return a.group <= 4 ? launch_gm<4, GEN>(a, s) : a.group <= 8 ? launch_gm<8, GEN>(a, s) : launch_gm<16, GEN>(a, s);
}

size_t attend_lds_bytes(int kbuf_words, int vbuf_words, int nbuf, int group) {
  const int gm = group <= 4 ? 4 : group <= 8 ? 8 : 16;
  return (64 + kWaves * 48 + kWaves * (size_t)wave_lds_words(kbuf_words, vbuf_words, nbuf, gm)) * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a_in, hipStream_t s) {
  AttendArgs a = a_in;
  if (a.n_tokens > 0) {
    // tile buffers: 64 records plus the 16-byte copy granule and one word read past the last record
    int wkm = 0, wvm = 0;
    bool gen = false;
    for (int h = 0; h < a.n_kv_heads; ++h) {
      const HeadDesc& d = a.heads.h[h];
      wkm = d.wk > wkm ? d.wk : wkm;
      wvm = d.wv > wvm ? d.wv : wvm;
      gen |= !(pow2_bits(d.bk) && pow2_bits(d.bv));
    }
    a.kbuf_words = ((64 * wkm + 4 + 3) / 4) * 4;
    a.vbuf_words = ((64 * wvm + 4 + 3) / 4) * 4;
    a.nbuf = attend_lds_bytes(a.kbuf_words, a.vbuf_words, 2, a.group) <= 160 * 1024 ? 2 : 1;
    // layouts whose widths are all powers of two use the instance without the general-width paths
    const hipError_t e = gen ? launch_widths<true>(a, s) : launch_widths<false>(a, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.n_kv_heads, (unsigned)a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvtc
