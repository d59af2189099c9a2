// Device building blocks of the split-K decode attention kernels (gfx950):
// record-tile streaming HBM -> LDS, the per-tile score / softmax / value phases
// on the matrix cores, and the workgroup and split merges.  Included by the
// generic kernel and by the kernels specialised per record format.
#pragma once

#include "encode_core.h"
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

// With GM = 4 the score MFMA packs the hi and lo query parts into rows [0, GM) and
// [GM, 2 GM) of one operand and leaves S[token][2 GM] (hi sums, then lo sums).  A
// doubled score area at GM = 8 would leave room for only two workgroups per CU on
// the mixed Qwen-shaped layout (137 µs against 88 µs), so GM = 8 puts the hi parts
// in rows [0, 8) and the lo parts in rows [8, 16), which land in lanes 32..63 of the
// result, and a lane swap across the two wave halves adds them to the hi sums
// before the store.
__host__ __device__ constexpr bool kpack(int gm) { return gm == 4; }
__host__ __device__ constexpr bool k_packed(int gm) { return gm <= 8; }
__host__ __device__ constexpr int k_lo_row(int gm) { return kpack(gm) ? gm : (k_packed(gm) ? 8 : 0); }
__host__ __device__ constexpr int score_floats(int gm) { return 64 * (kpack(gm) ? 2 * gm : gm); }
__host__ __device__ constexpr int score_words(int gm) { return score_floats(gm) + 4; }  // + the zero slot

// One v_permlane32_swap folds two values: lane l < 32 returns x[l] + x[l + 32] and
// lane l >= 32 returns y[l - 32] + y[l].  The empty asm hands the builtin opaque
// scalars: fed straight from vector elements, this compiler lowers every such swap
// on element 0 of the vector.
__device__ inline float fold_halves(float x, float y) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = __builtin_bit_cast(uint32_t, y);
  asm volatile("" : "+v"(a), "+v"(b));
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

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
template <int CTRL>
__device__ inline float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
  return x + __builtin_bit_cast(float, y);
}
// Wave-uniform sum: DPP within rows of 16 lanes, then the four row results.
__device__ inline float wave_sum_uniform(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);  // row_half_mirror
  x = dpp_add<0x140>(x);  // row_mirror
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return (r0 + r1) + (r2 + r3);
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
// Buffer resource of a cache region as four SGPRs: base, stride 0, byte size
// (out-of-range offsets read zero), raw 32-bit dword format.
typedef u32x4 rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// One 16-byte-per-lane buffer load straight into LDS: lane l's bytes land at
// lds + 16*l.  Written as asm so that the compiler does not treat it as an LDS
// store and wait for it before every later LDS read: the tile loop orders these
// copies with explicit vmcnt waits instead.  M0 carries the LDS base; one wait
// state separates its write from the load that reads it.  The records are read
// once per launch, so the load is marked non-temporal: it does not push the
// bases, queries and split partials (read by every workgroup, or across
// workgroups) out of the caches (~4-5 us per launch at 128K).
__device__ inline void dma16(rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}

// Copy `nbytes` starting at byte `src` of the region to LDS `dst` in 16-byte
// chunks (up to 12 bytes past the end are copied too); issues copy_insts(nbytes)
// vector-memory instructions.
__device__ inline void tile_copy(rsrc_t r, uint32_t src, uint32_t nbytes, uint32_t base) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t n16 = (nbytes + 15u) >> 4;
  uint32_t c = 0;
  for (; c + 64 <= n16; c += 64) dma16(r, base + 16u * c, src + 16u * (c + lane));
  if (c + lane < n16)  // tail: only the lanes whose 16 bytes belong to the tile
    dma16(r, base + 16u * c, src + 16u * (c + lane));
}
__device__ inline void tile_copy(rsrc_t r, uint32_t src, uint32_t nbytes, uint32_t* dst) {
  tile_copy(r, src, nbytes, lds_addr(dst));
}

// tile_copy of a compile-time size: the 64-lane chunks unrolled, then the tail.
template <uint32_t NBYTES>
__device__ inline void tile_copy_n(rsrc_t r, uint32_t src, uint32_t* dst) {
  constexpr uint32_t n16 = (NBYTES + 15u) >> 4;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t base = lds_addr(dst);
#pragma unroll
  for (uint32_t c = 0; c + 64 <= n16; c += 64) dma16(r, base + 16u * c, src + 16u * (c + lane));
  if constexpr (n16 % 64 != 0) {
    constexpr uint32_t c = n16 / 64 * 64;
    if (c + lane < n16) dma16(r, base + 16u * c, src + 16u * (c + lane));
  }
}

__device__ inline void wait_tiles() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory instructions of this wave are outstanding.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Vector-memory instructions tile_copy issues for `nbytes`.
__device__ inline int copy_insts(uint32_t nbytes) { return (int)((((nbytes + 15u) >> 4) + 63u) >> 6); }

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

// General widths: the NA words of a lane's code span that starts at stream bit
// `sb` (p: the record's first code word), read once and shifted so that the span
// begins at bit 0 of a[0].  ALIGNED: sb is a multiple of 32 for every lane.
template <int NA, bool ALIGNED>
__device__ __attribute__((always_inline)) inline void span_words(const uint32_t* p, int sb, uint32_t (&a)[NA]) {
  const uint32_t* q = p + (sb >> 5);
  if constexpr (ALIGNED) {
#pragma unroll
    for (int i = 0; i < NA; ++i) a[i] = q[i];
  } else {
    uint32_t w[NA + 1];
#pragma unroll
    for (int i = 0; i <= NA; ++i) w[i] = q[i];
#pragma unroll
    for (int i = 0; i < NA; ++i) a[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sb & 31);
  }
}

// Code c (B bits at bit c B) of a span held in registers; c is a constant once the
// callers' loops are unrolled, so the word index and shift fold away.  No code of
// a span reaches past its last word (the span is a whole number of codes), so the
// clamp of the second index only keeps the untaken branch in range.
template <int B, int NA>
__device__ __attribute__((always_inline)) inline uint32_t span_code(const uint32_t (&a)[NA], int c) {
  const int bit = c * B, wd = bit >> 5, off = bit & 31;
  if (off + B <= 32) return (a[wd] >> off) & ((1u << B) - 1u);
  return __builtin_amdgcn_alignbit(a[wd + 1 < NA ? wd + 1 : wd], a[wd], off) & ((1u << B) - 1u);
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

// k_slot with the width known only at run time (generic kernel).
__device__ inline void k_slot_rt(int B, int G, int nks, int ks, int p, int rk, bool& valid, int& j_lo, int& j_hi,
                                 int& s) {
  const int pi = G * nks * 4 + ks * 4 + p;
  valid = pi < rk / 2;
  if (pow2_bits(B)) {
    const int ppw = 16 / B;
    const int w = pi / ppw, u = pi % ppw;
    j_lo = w * (32 / B) + u;
    j_hi = j_lo + ppw;
    const int o = ((ks * 4 + p) % ppw) * B;
    s = o + B <= 10 ? o : o - (B == 2 ? 10 : 8);
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
                                                              float* S, const uint32_t* cb = nullptr) {
  // tokens past the tile's last record read stale LDS: their codes are finite and
  // their scores are replaced by -inf before the softmax.  The four 16-token
  // sub-tiles are interleaved so that consecutive MFMAs never depend on each other.
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  const uint32_t* rec0 = kt + n * wk;
  f32x4 acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    constexpr int NWL = (NKS * 4 * B + 15) / 16;
    const int base = G * NKS * 4;
    uint32_t w[4][NWL];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      lds_words<NWL>(rec0 + tt * 16 * wk + 1 + base / PPW, w[tt]);
      if constexpr (NKS * 4 < PPW) w[tt][0] >>= (base % PPW) * B;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 bop[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int pl = ks * 4 + p;
          bop[tt][p] = Pow2<B>::pair(w[tt][pl / PPW], (pl % PPW) * B);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_hi[ks], bop[tt], acc[tt]);
      if constexpr (!k_packed(GM)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_lo[ks], bop[tt], acc[tt]);
      }
    }
  } else if constexpr (is_vq(B)) {
    // vector-quantized pairs: lane group G holds pairs [4 NKS G, 4 NKS (G + 1)) of each
    // token (pair slot p of K-step ks is pair pi = 4 NKS G + 4 ks + p, coordinates 2 pi
    // and 2 pi + 1), one b-bit index each; the operand dword is the pair's codeword
    // from the LDS codebook cb ([pair][2^b], fp16 even | odd << 16): normal fp16
    // values, so the key scale carries no 2^24 (see project_query)
    constexpr int BI = code_bits(B);
    constexpr int SPAN = 4 * NKS * BI;
    constexpr int NA = (SPAN + 31) / 32;
    uint32_t a[4][NA];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) span_words<NA, SPAN % 32 == 0>(rec0 + tt * 16 * wk + 1, G * SPAN, a[tt]);
    constexpr int SK = vq_kstride(B, 32 * NKS);  // padded row stride: the lane groups read different banks
    const uint32_t* cbg = cb + G * 4 * NKS * SK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 bop[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int p = 0; p < 4; ++p) bop[tt][p] = cbg[(4 * ks + p) * SK + span_code<BI>(a[tt], 4 * ks + p)];
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_hi[ks], bop[tt], acc[tt]);
      if constexpr (!k_packed(GM)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_lo[ks], bop[tt], acc[tt]);
      }
    }
  } else {
    // lane group G holds codes [8 NKS G, 8 NKS (G + 1)) of each token: read once
    constexpr int SPAN = 8 * NKS * B;
    constexpr int NA = (SPAN + 31) / 32;
    uint32_t a[4][NA];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) span_words<NA, SPAN % 32 == 0>(rec0 + tt * 16 * wk + 1, G * SPAN, a[tt]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 bop[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          bop[tt][p] = span_code<B>(a[tt], 8 * ks + 2 * p) | (span_code<B>(a[tt], 8 * ks + 2 * p + 1) << 16);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_hi[ks], bop[tt], acc[tt]);
      if constexpr (!k_packed(GM)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma(aq_lo[ks], bop[tt], acc[tt]);
      }
    }
  }
  if constexpr (k_packed(GM) && !kpack(GM)) {
    // S[token][8]: tiles 2u and 2u + 1 folded together, the low wave half storing
    // tile 2u and the high half tile 2u + 1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = fold_halves(acc[2 * u][e], acc[2 * u + 1][e]);
      *(f32x4*)(S + ((2 * u + (G >> 1)) * 16 + n) * GM + 4 * (G & 1)) = r;
    }
    return;
  }
  // S[token][GM] (GM = 4: S[token][2][GM], the hi rows then the lo rows): the lanes
  // of the all-zero rows store nothing
  constexpr int kRows = kpack(GM) ? 2 * GM : GM;
  if (4 * G < kRows) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) *(f32x4*)(S + (tt * 16 + n) * kRows + 4 * G) = acc[tt];
  }
}

// One 32-token value step (tile tokens 32*kk .. 32*kk+31): for each N-tile of 16
// codes the B operand (lane n owns codes [n*NT, (n+1)*NT) of the 8 tokens of its
// lane group, one aligned field of NT*B bits for power-of-two widths) and its MFMAs
// with A = p*step_V.  PACK (g <= 8): the hi and lo fp16 parts of A sit in rows
// [0, GM) and [GM, 2 GM) of one operand, one MFMA per N-tile, and the two row
// blocks of the accumulator are added at the end; otherwise two MFMAs (hi, lo).
template <int B, int NT, bool PACK>
__device__ __attribute__((always_inline)) inline void v_phase(const uint32_t* vt, int wv, int kk,
                                                              u32x4 ahi, u32x4 alo, f32x4 (&acc2)[8],
                                                              const uint32_t* cb = nullptr) {
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
    // N-tiles in pairs: both hi MFMAs, then both lo MFMAs (no back-to-back dependency)
#pragma unroll
    for (int n2 = 0; n2 < NT; n2 += 2) {
      u32x4 bop[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int nt = n2 + u < NT ? n2 + u : NT - 1;
        const int k = nt / PPW;  // 16-bit slice of the field
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t fa = k < 2 ? f0[2 * p] : f1[2 * p];
          const uint32_t fb = k < 2 ? f0[2 * p + 1] : f1[2 * p + 1];
          const uint32_t y = (k & 1) ? ((fa >> 16) | (fb & 0xFFFF0000u)) : ((fa & 0xFFFFu) | (fb << 16));
          bop[u][p] = Pow2<B>::pair(y, (nt % PPW) * B);
        }
      }
      acc2[n2] = mfma(ahi, bop[0], acc2[n2]);
      if (n2 + 1 < NT) acc2[n2 + 1] = mfma(ahi, bop[1], acc2[n2 + 1]);
      if constexpr (!PACK) {
        acc2[n2] = mfma(alo, bop[0], acc2[n2]);
        if (n2 + 1 < NT) acc2[n2 + 1] = mfma(alo, bop[1], acc2[n2 + 1]);
      }
    }
  } else if constexpr (is_vq(B)) {
    // vector-quantized pairs: lane column block n holds pairs [n NT/2, (n + 1) NT/2) of
    // each of its 8 tokens; N-tiles 2u and 2u + 1 take the even and odd coordinate of
    // pair n NT/2 + u, so that column n of N-tile nt is coordinate n NT + nt as with
    // scalar codes.  One LDS codebook read per (token, pair) serves both N-tiles.
    static_assert(NT % 2 == 0, "vector-quantized values need r_V >= 32");
    constexpr int BI = code_bits(B);
    constexpr int FS = (NT / 2) * BI;
    constexpr int NA = (FS + 31) / 32;
    uint32_t a[8][NA];
#pragma unroll
    for (int e = 0; e < 8; ++e) span_words<NA, FS % 32 == 0>(rec0 + e * wv, n * FS, a[e]);
    constexpr int SV = vq_vstride(B);
    const uint32_t* cbn = cb + n * (NT / 2) * SV;
#pragma unroll
    for (int u = 0; u < NT / 2; ++u) {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = cbn[u * SV + span_code<BI>(a[e], u)];
      u32x4 b0, b1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // byte permutes: the low halves, then the high halves, of tokens 2p, 2p + 1
        b0[p] = __builtin_amdgcn_perm(w[2 * p + 1], w[2 * p], 0x05040100u);
        b1[p] = __builtin_amdgcn_perm(w[2 * p + 1], w[2 * p], 0x07060302u);
      }
      acc2[2 * u] = mfma(ahi, b0, acc2[2 * u]);
      acc2[2 * u + 1] = mfma(ahi, b1, acc2[2 * u + 1]);
      if constexpr (!PACK) {
        acc2[2 * u] = mfma(alo, b0, acc2[2 * u]);
        acc2[2 * u + 1] = mfma(alo, b1, acc2[2 * u + 1]);
      }
    }
  } else {
    // lane column block n holds codes [n NT, (n + 1) NT) of each of its 8 tokens: read once
    constexpr int FS = NT * B;
    constexpr int NA = (FS + 31) / 32;
    uint32_t a[8][NA];
#pragma unroll
    for (int e = 0; e < 8; ++e) span_words<NA, FS % 32 == 0>(rec0 + e * wv, n * FS, a[e]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      u32x4 bop;
#pragma unroll
      for (int p = 0; p < 4; ++p) bop[p] = span_code<B>(a[2 * p], nt) | (span_code<B>(a[2 * p + 1], nt) << 16);
      acc2[nt] = mfma(ahi, bop, acc2[nt]);
      if constexpr (!PACK) acc2[nt] = mfma(alo, bop, acc2[nt]);
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

// LDS of an attend workgroup, in 32-bit words:
//   common: per wave m[16] l[16] c[16]; a flag word (padded); per head E, sum(q~), 2^(24-E)
//   scores: per wave S[64][GM] (fp32; S[64][2][GM] hi and lo sums for GM = 4),
//           overwritten by the probabilities
//           P[2][GM][64] (fp16, hi then lo) once read, and a 4-word zero slot read
//           as the A rows >= GM; before the tile loop the whole region holds the
//           query staging of the projection (q[g][128], q~[g][128])
//   tiles:  per wave nbuf K and nbuf V record tiles; at the end the wave's value
//           partial o~[g][r_V], then the split merge's o~[g][128]
__host__ __device__ inline int tile_lds_words(int kbuf_words, int vbuf_words, int nbuf, int gm) {
  const int w = nbuf * (kbuf_words + vbuf_words);
  const int part = (gm <= 8 ? 2 : 1) * gm * kMaxRank;  // the wave's value partial (hi and lo rows when packed)
  return w > part ? w : part;
}
// LDS words of the RoPE kernel's exchange (after the tile areas): the partial scores
// [source wave][tile of wave][64 tokens][GM] of one step; the 128 row sums of the key
// basis; (cos, sin) of 16 theta_i per pair; the 64 inverse frequencies (float64); and
// each wave's query operands [wave][lane][8].
__host__ __device__ constexpr int rope_lds_words(int gm) {
  return kWaves * kWaves * kTileT * gm + kHeadDim + kHeadDim + kHeadDim + kWaves * 64 * 8;
}

constexpr int kHeadStats = 3 * kMaxGroup;
constexpr int kCommonWords = kWaves * 48 + 4 + kHeadStats;

// The fused append encodes K and V with one EncodeScratch each in the score and
// tile areas, which are at least this large for every group size.
static_assert(2 * sizeof(EncodeScratch) <= sizeof(float) * kWaves * (size_t)(score_words(4) + 4 * kMaxRank),
              "encode scratch does not fit the score and tile areas");
static_assert(kCommonWords % 2 == 0, "encode scratch (float64) must start 8-byte aligned");

// Dynamic LDS bytes of an attend workgroup.
__host__ __device__ inline size_t attend_lds_bytes(int kbuf_words, int vbuf_words, int nbuf, int group) {
  const int gm = group <= 4 ? 4 : group <= 8 ? 8 : 16;
  return (kCommonWords + kWaves * (size_t)(score_words(gm) + tile_lds_words(kbuf_words, vbuf_words, nbuf, gm))) *
         sizeof(float);
}

// ----------------------------------------------------------------- split merge
// Split partials cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other): they are written and read as relaxed device-scope atomics, which
// bypass the non-coherent cache level, and ordered by the arrival counter after
// each writer has waited for its stores to complete.  This avoids the whole-cache
// write-back and invalidate of device-scope fences.
__device__ inline void part_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void part_store_u32(float* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float part_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two adjacent partial floats (8-byte aligned) in one coherent load.
__device__ inline void part_load2(const float* p, float& x, float& y) {
  const uint64_t v = __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  x = __builtin_bit_cast(float, (uint32_t)v);
  y = __builtin_bit_cast(float, (uint32_t)(v >> 32));
}
// Offsets in a split partial: o[0, 128) (the back-projected P_V o~ of the split,
// unnormalised), then m, l and the tag of the call that wrote it (the call's
// nonce, stored with m and l before the split's arrival is counted).
constexpr int kPartM = kMaxRank, kPartL = kMaxRank + 1, kPartTag = kMaxRank + 2;
static_assert(kPartTag + 1 < kPartStride, "split partial layout");

constexpr int kMergeChunk = 16;  // splits whose loads one merging thread has in flight (one round up to 32 splits)

// Run by a workgroup that arrived as the last of the ns splits of a (sequence, KV
// head), or later (only with a counter that was not zero on entry), to finish the
// split partials.  Work item = (head, 4 consecutive output dimensions); with at
// most 128 items two threads share one, each taking every other kMergeChunk
// splits.  A thread issues the coherent loads of kMergeChunk splits (output quad,
// m, l and tag) at once and folds them into a running log-sum-exp; the two halves
// combine through a lane exchange and o / l is the output (the back-projection
// already happened in each split's workgroup, since it commutes with the weighted
// sum).  An item for which any split's tag is not this call's nonce (a partial
// not yet written by this call: possible only when the counter started above
// zero, so that a workgroup counted as last before every split had arrived) gets
// NaN instead.  Every merge of an item over the same partials writes the same
// bits, so the output is correct or NaN, never a fold of a stale partial.  The
// workgroup that arrived exactly ns-th (reset = true) leaves the counter at zero
// for the next call.
__device__ inline void merge_splits(const AttendArgs& a, int h, int b, bool reset) {
  const int tid = threadIdx.x;
  const int g = a.group, ns = head_desc(a.heads, h).ns;
  const int64_t bq0 = (int64_t)b * a.n_q_heads + (int64_t)h * g;
  // item = (query head, four output dimensions); two threads per item when they fit
  const int items = g * (kHeadDim / 4);
  const int tpi = items <= 128 ? 2 : 1;
  for (int t0 = 0; t0 < items * tpi; t0 += 256) {
    const int t = t0 + tid;
    const int item = t / tpi, sp = t % tpi;  // sp: which splits of the item this thread takes
    const int hh = item / (kHeadDim / 4), jq = item % (kHeadDim / 4);
    const bool act = item < items;
    const float* part = a.part + (bq0 + (act ? hh : 0)) * a.n_splits * (int64_t)kPartStride + 4 * jq;
    float M = -__builtin_inff(), L = 0.0f, A0 = 0.0f, A1 = 0.0f, A2 = 0.0f, A3 = 0.0f;
    bool stale = false;
    for (int s0 = kMergeChunk * sp; s0 < ns; s0 += kMergeChunk * tpi) {
      float o[kMergeChunk][4], mv[kMergeChunk], lv[kMergeChunk];
      uint32_t tg[kMergeChunk];
      // every load unconditional (splits past the last one re-read it and get weight
      // 0), so that all of them are in flight before the first wait
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        const int sk = s0 + k < ns ? s0 + k : ns - 1;
        const float* ps = part + (int64_t)sk * kPartStride;
        part_load2(ps, o[k][0], o[k][1]);
        part_load2(ps + 2, o[k][2], o[k][3]);
        part_load2(ps - 4 * jq + kPartM, mv[k], lv[k]);
        tg[k] = __hip_atomic_load((uint32_t*)const_cast<float*>(ps - 4 * jq + kPartTag), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        stale |= tg[k] != a.nonce;
        if (s0 + k >= ns) mv[k] = -__builtin_inff();
      }
      float mc = M;
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) mc = fmaxf(mc, mv[k]);
      const float mu = mc == -__builtin_inff() ? 0.0f : mc;  // empty splits carry m = -inf, weight 0
      const float sc = exp2f(M - mu);
      L *= sc;
      A0 *= sc;
      A1 *= sc;
      A2 *= sc;
      A3 *= sc;
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        const float wgt = exp2f(mv[k] - mu);
        L = fmaf(wgt, lv[k], L);
        A0 = fmaf(wgt, o[k][0], A0);
        A1 = fmaf(wgt, o[k][1], A1);
        A2 = fmaf(wgt, o[k][2], A2);
        A3 = fmaf(wgt, o[k][3], A3);
      }
      M = mc;
    }
    if (tpi == 2) {  // the two halves of an item sit in adjacent lanes
      const float Mo = __shfl_xor(M, 1);
      const float Mx = fmaxf(M, Mo);
      const float mu = Mx == -__builtin_inff() ? 0.0f : Mx;
      const float sc = exp2f(M - mu);
      L *= sc;
      A0 *= sc;
      A1 *= sc;
      A2 *= sc;
      A3 *= sc;
      L += __shfl_xor(L, 1);
      A0 += __shfl_xor(A0, 1);
      A1 += __shfl_xor(A1, 1);
      A2 += __shfl_xor(A2, 1);
      A3 += __shfl_xor(A3, 1);
      stale |= __shfl_xor((int)stale, 1) != 0;
    }
    if (act && sp == 0) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float nan = __builtin_nanf("");
      const f32x4 r = stale ? f32x4{nan, nan, nan, nan} : f32x4{A0 * inv, A1 * inv, A2 * inv, A3 * inv};
      *(f32x4*)(a.out + (bq0 + hh) * kHeadDim + 4 * jq) = r;
    }
  }
  if (tid == 0 && reset)
    __hip_atomic_store(a.cnt + (int64_t)b * a.n_kv_heads + h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- phase stamps (diagnostic builds)
// Built with KVTC_STAMPS, the kernels record the 100 MHz real-time counter at the
// phase boundaries of every workgroup into the caller's stamp buffer (kStampWords
// 64-bit words per workgroup): 0 entry, 1 query projection done (wave 0), 2-5 tile
// loop done per wave, 6 split partial stored, 7 arrival counted, 8 split merge done
// (merging workgroup only), 9 hardware id, 10 XCC id, 11 fused append done, 12 wave
// partials staged in LDS, 13 wave merge done, 14 back-projection stored (issued),
// 16-19 per wave: its partial written to LDS, 20-23 per wave: its P_V row loads issued;
// query projection (wave 0): 28 start, 24 loads and first copies issued, 25 queries
// staged, 26 projected, 27 exponents and sums done; set-up: 29 head found, 30 split
// bounds, 31 buffers set (before the fused append).
// Other builds compile none of it.
constexpr int kStampWords = 32;
#ifdef KVTC_STAMPS
#define KVTC_STAMP(ptr, i)                                            \
  do {                                                                \
    if (ptr) (ptr)[i] = (uint64_t)__builtin_amdgcn_s_memrealtime();   \
  } while (0)
#else
#define KVTC_STAMP(ptr, i) \
  do {                     \
  } while (0)
#endif

// ----------------------------------------------------------------- wave state and context
// Running state of one wave: reference maximum, per-lane partial sums of p and
// p * min_V per head, and the value accumulators of up to 8 N-tiles (lane (n, G)
// holds heads 4G..4G+3 of codes n*NT + nt).
template <int GM>
struct WaveState {
  float m[GM], l[GM], c[GM];
  f32x4 acc2[8];
};

// What a wave's tile loop needs of the kernel prologue.
struct WaveCtx {
  rsrc_t rk_, rv_;          // cache regions of this (sequence, KV head)
  uint32_t* ktile;          // [nbuf][kbuf] K record tiles
  uint32_t* vtile;          // [nbuf][vbuf] V record tiles
  float* S;                 // scores, then probabilities, then the zero slot
  float* stage;             // the workgroup's score region: query staging before the tile loop
  float* stats;             // per head E, sum(q~), 2^(24-E)
  int kbuf, vbuf, nbuf;
  int t_begin, t_end;       // this wave's tokens
  int g;
  int h, b;                 // KV head and sequence of this workgroup
  int64_t unit;             // sequence * n_kv_heads + KV head
  uint64_t* stamp;          // this workgroup's phase stamps (diagnostic builds), else null
  const int32_t* bt_row;    // paged: this sequence's block-table row, else null
  int page;                 // paged: tokens per page
  uint32_t pool_recs;       // paged: records in a head's pool (an offset past them reads zeros)
  int64_t pool_pages;
  const uint32_t* cbk;      // vector-quantized records: the head's K / V codebooks in LDS, else null
  const uint32_t* cbv;
  int split_begin;          // the split's first token; wave w streams [split_begin + w wave_tokens, + wave_tokens)
  int wave_tokens;          //   clipped to n_tok
  int n_tok;                // this sequence's context length
  int wave_area;            // LDS words of one wave's record tiles (wave w's tiles at ktile + (w - wave) wave_area)
  float* extra;             // LDS after the tile areas (codebooks, or the exchange of the RoPE kernel)
};

// Record index, within the buffer resource of the wave's cache regions, of the tile
// that starts at token t0 (a multiple of 64: a tile never crosses a page): t0 for
// contiguous records, its pool slot for paged ones (past the pool, so that the copy
// reads zeros, for a block-table entry outside it).
__device__ inline uint32_t tile_rec(const WaveCtx& c, int t0) {
  if (!c.bt_row) return (uint32_t)t0;
  const int p = __builtin_amdgcn_readfirstlane(c.bt_row[t0 / c.page]);
  if (p < 0 || (int64_t)p >= c.pool_pages) return c.pool_recs;
  return (uint32_t)p * (uint32_t)c.page + (uint32_t)(t0 % c.page);
}

// Key operand (A of the score MFMA) for one (K-step, lane): row = head (lane % 16),
// element of pair slot = q~_j * 2^(E_head - s), split into fp16 hi + lo.  PACK =
// GM (GM <= 8): one operand, rows [0, GM) the hi and rows [GM, 2 GM) the lo parts
// (returned in `hi`); PACK = 0: separate hi and lo operands.  B = 0: the width bk
// is known only at run time.
template <int B, int PACK>
__device__ inline void aq_slot(const float* qt, const float* E_h, int g, int rk, int bk, int ks, int lane,
                               u32x4& hi, u32x4& lo) {
  const int r16 = lane & 15, G = lane >> 4;
  const int i = PACK ? (r16 & (PACK - 1)) : r16;  // the head of this row
  const bool row_on = PACK ? r16 < 2 * PACK : true;
  const bool lo_row = PACK && r16 >= PACK;
  const int nks = rk >= 32 ? rk / 32 : 1;
  const int E = i < g ? (int)E_h[i] : 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    bool valid;
    int jl, jh, sh;
    if constexpr (B == 0) k_slot_rt(bk, G, nks, ks, p, rk, valid, jl, jh, sh);
    else k_slot<B>(G, nks, ks, p, rk, valid, jl, jh, sh);
    float xl = 0.0f, xh = 0.0f;
    if (valid && row_on && i < g && ks < nks) {
      xl = ldexpf(qt[i * kMaxRank + jl], E - sh);
      xh = ldexpf(qt[i * kMaxRank + jh], E - sh);
    }
    const _Float16 hl = (_Float16)xl, hh = (_Float16)xh;
    const _Float16 ll = (_Float16)(xl - (float)hl), lh = (_Float16)(xh - (float)hh);
    const uint32_t hw = h2u(hl) | (h2u(hh) << 16), lw = h2u(ll) | (h2u(lh) << 16);
    hi[p] = lo_row ? lw : hw;
    lo[p] = lw;
  }
}

// The g query heads of this KV head projected into its key basis by the whole
// workgroup, q~ = scale * log2(e) * Q_K^T q (the inverse key transform folded into
// the query; Q_K is the query-side key basis, P_K itself when orthonormal), while
// the first record tiles stream in: the queries and the basis
// columns are requested first, then `issue` starts the first tile copies, then the
// arithmetic waits for its loads (the memory counter completes in order, so only
// the last basis loads also wait for the copies, which were issued right behind
// them).  Wave w owns columns
// [w r_K / 4, (w+1) r_K / 4) of P_K; its lanes split the 128 rows into groups
// (each lane loads its column segment once and serves all g heads), and the row
// groups are summed across lanes.  Then per head the exponent E (max |q~| 2^E <
// 2^14), sum(q~) and 2^(24-E), and each wave's MFMA A operands of q~ (B: the key
// code width as unpacked by the score phase, 0 to read it from the head at run time).
template <int GM, int B, class Issue>
__device__ __attribute__((always_inline)) inline void project_query(const AttendArgs& a, const WaveCtx& c, int rk,
                                                                    u32x4 (&aq_hi)[4], u32x4 (&aq_lo)[4],
                                                                    float (&sq)[GM], float (&kf)[GM],
                                                                    Issue&& issue) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = c.h, b = c.b, g = c.g;
  const HeadDesc hd = head_desc(a.heads, h);
  const int64_t bq0 = (int64_t)b * a.n_q_heads + (int64_t)h * g;
  float* qs = c.stage;                    // [128][GM] raw queries, row-major over the head dimension
  float* qt = c.stage + GM * kHeadDim;    // [g][kMaxRank] projected
  const int cw = rk / 4;                  // columns per wave
  const int rg = 64 / cw;                 // row groups per column
  const int rpg = kHeadDim / rg;          // rows per group (r_K / 2)
  const int jj = lane % cw, rgi = lane / cw;
  const int j = wave * cw + jj;
  if (tid == 0) KVTC_STAMP(c.stamp, 28);
  const float* col = a.basis_k + hd.qoff_k + (int64_t)(rgi * rpg) * rk + j;
  // every load in flight before the first use: the queries (used first), then the
  // column segment, then the first tile copies
  constexpr int kQ = GM * kHeadDim / 256;
  float qv[kQ];
#pragma unroll
  for (int k = 0; k < kQ; ++k) {
    const int idx = tid + 256 * k;
    qv[k] = 0.0f;
    if (idx < g * kHeadDim) {
      const int64_t off = bq0 * kHeadDim + idx;
      qv[k] = a.dtype == 0 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off];
    }
  }
  float pk[kMaxRank / 2];
#pragma unroll
  for (int k = 0; k < kMaxRank / 2; ++k)
    if (k < rpg) pk[k] = col[(int64_t)k * rk];
  issue();
  if (tid == 0) KVTC_STAMP(c.stamp, 24);
#pragma unroll
  for (int k = 0; k < kQ; ++k) {
    const int idx = tid + 256 * k;  // head idx / 128, dimension idx % 128
    qs[(idx % kHeadDim) * GM + idx / kHeadDim] = qv[k];
  }
  __syncthreads();
  if (tid == 0) KVTC_STAMP(c.stamp, 25);
  for (int h4 = 0; h4 < g; h4 += 4) {  // four heads at a time; the column segment stays in registers
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxRank / 2; ++k) {
      if (k < rpg) {
        const f32x4 qq = *(const f32x4*)(qs + (rgi * rpg + k) * GM + h4);
        acc[0] = fmaf(pk[k], qq[0], acc[0]);
        acc[1] = fmaf(pk[k], qq[1], acc[1]);
        acc[2] = fmaf(pk[k], qq[2], acc[2]);
        acc[3] = fmaf(pk[k], qq[3], acc[3]);
      }
    }
    for (int off = cw; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (rgi == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (h4 + e < g) qt[(h4 + e) * kMaxRank + j] = acc[e] * a.scale_log2;
    }
  }
  __syncthreads();
  if (tid == 0) KVTC_STAMP(c.stamp, 26);
  float* Eh = c.stats;
  for (int hh = wave; hh < g; hh += kWaves) {  // one wave per head: sum and max |q~| over the rank
    const float v0 = lane < rk ? qt[hh * kMaxRank + lane] : 0.0f;
    const float v1 = lane + 64 < rk ? qt[hh * kMaxRank + lane + 64] : 0.0f;
    const float sum = wave_sum_uniform(v0 + v1);  // DPP row reductions: no LDS round trips
    const float mx = wave_max_uniform(fmaxf(fabsf(v0), fabsf(v1)));
    int e = 0;
    if (mx > 0.0f) {
      frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
      e = 14 - e;      // max |q~| * 2^E < 2^14
    }
    if (lane == 0) {
      Eh[hh] = (float)e;
      Eh[kMaxGroup + hh] = sum;
      Eh[2 * kMaxGroup + hh] = ldexpf(1.0f, (is_vq(hd.bk) ? 0 : 24) - e);  // codes: subnormal fp16 operands
    }
  }
  __syncthreads();
  if (tid == 0) KVTC_STAMP(c.stamp, 27);
  const int nks = rk >= 32 ? rk / 32 : 1;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < nks) {
      aq_slot<B, k_lo_row(GM)>(qt, Eh, g, rk, hd.bk, ks, lane, aq_hi[ks], aq_lo[ks]);
    } else {
      aq_hi[ks] = u32x4{0u, 0u, 0u, 0u};
      aq_lo[ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    sq[hh] = hh < g ? uniform(Eh[kMaxGroup + hh]) : 0.0f;
    kf[hh] = hh < g ? uniform(Eh[2 * kMaxGroup + hh]) : 0.0f;
  }
  __syncthreads();  // the staging region becomes the waves' score areas
}

template <int GM>
__device__ __attribute__((always_inline)) inline void init_state(WaveState<GM>& st) {
  // finite start, so heads >= g never form -inf - -inf
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    st.m[hh] = -1e30f;
    st.l[hh] = 0.0f;
    st.c[hh] = 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) st.acc2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Waves of a CU issue by age, so the workgroups resident first finish their splits
// early and the last ones run their final tiles at lower occupancy.  Each wave
// raises its issue priority with the share of its tokens still ahead of it (3 in
// the first quarter, then 2, 1, 0), so the waves that are behind catch up and all
// finish together.  Comparisons only: a division here costs ~25 scalar
// instructions per tile.
__device__ inline void progress_priority(int t0, int t_begin, int t_end) {
  const int q = t_end - t_begin, d = t0 - t_begin;
  if (4 * d < q) __builtin_amdgcn_s_setprio(3);
  else if (2 * d < q) __builtin_amdgcn_s_setprio(2);
  else if (4 * d < 3 * q) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Online softmax of one tile, one token per lane (branch-free over heads), after
// the score phase has left S[token][GM]: s = min_K * sum(q~) + step_K 2^(24-E) S
// (log2 units).  Each head keeps a reference M that bounds the log2 value weight
// u = s + log2(step_V) of every token seen (step_V clamped to >= 2^-24), so that
// x = 2^kPScale * 2^(s - M) * step_V <= 2^kPScale: the value operand P = x (fp16
// hi + lo) neither overflows nor, for tokens within 2^-28 of the heaviest one,
// leaves the normal fp16 range.  M moves lazily: only when a token exceeds it, and
// then to the tile's maximum plus kLazyMargin, so that later tiles rarely move it.
// p = 2^(s - M) <= 2^24 feeds the fp32 sums l and c.  hk / hv = 0: the key /
// value records are header-free and every token takes the head's fixed min and
// step sk / sv (fp16 min | fp16 step << 16).
constexpr int kPScale = 14;
constexpr float kLazyMargin = 8.0f;

template <int GM>
__device__ __attribute__((always_inline)) inline void softmax_tile(const uint32_t* kt, const uint32_t* vt, int wk,
                                                                   int wv, int hk, int hv, uint32_t sk, uint32_t sv,
                                                                   int nvalid, int g, float* S,
                                                                   const float (&sq)[GM], const float (&kf)[GM],
                                                                   WaveState<GM>& st) {
  const int lane = threadIdx.x & 63, G = lane >> 4;
  _Float16* P = (_Float16*)S;
  const bool valid = lane < nvalid;
  const uint32_t kh = hk ? kt[lane * wk] : sk;
  const uint32_t vh = hv ? vt[lane * wv] : sv;
  const float muk = f16_bits_to_f32(kh & 0xFFFFu), sgk = f16_bits_to_f32(kh >> 16);
  const float muv = valid ? f16_bits_to_f32(vh & 0xFFFFu) : 0.0f;
  const float sgv = valid ? f16_bits_to_f32(vh >> 16) : 0.0f;
  const float lsg = __builtin_amdgcn_logf(fmaxf(sgv, 0x1p-24f));  // log2 of the clamped step
  const float sgx = sgv * (float)(1 << kPScale);
  lds_fence();
  float s[GM], u[GM];
#pragma unroll
  for (int q4 = 0; q4 < GM / 4; ++q4) {
    f32x4 d;
    if constexpr (kpack(GM)) {  // hi sums + lo sums
      const f32x4 dh = *(const f32x4*)(S + lane * 2 * GM + 4 * q4);
      const f32x4 dl = *(const f32x4*)(S + lane * 2 * GM + GM + 4 * q4);
      d = dh + dl;
    } else {
      d = *(const f32x4*)(S + lane * GM + 4 * q4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hh = 4 * q4 + e;
      const float x = fmaf(sgk * kf[hh], d[e], muk * sq[hh]);
      s[hh] = (valid && hh < g) ? x : -__builtin_inff();
      u[hh] = s[hh] + lsg;
    }
  }
  bool up = false;
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) up |= u[hh] > st.m[hh];
  if (__any(up)) {
    float alpha[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      const float mx = wave_max_uniform(u[hh]);
      const float mn = mx > st.m[hh] ? mx + kLazyMargin : st.m[hh];
      alpha[hh] = exp2f(st.m[hh] - mn);  // 1 if unchanged, 0 on the first tile
      st.m[hh] = mn;
      st.l[hh] *= alpha[hh];
      st.c[hh] *= alpha[hh];
    }
    // value accumulators: lane (n, G) holds heads 4G..4G+3; alpha through LDS
    lds_fence();
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) S[hh] = alpha[hh];
    }
    lds_fence();
    // lane group G holds accumulator rows 4G..4G+3: heads 4G.. (hi), or with packed
    // value operands (GM <= 8) rows GM..2GM-1 are the lo parts of heads 0..GM-1
    constexpr int kRows = GM <= 8 ? 2 * GM : GM;
    const f32x4 f = 4 * G < kRows ? *(const f32x4*)(S + ((4 * G) & (GM - 1))) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.acc2[nt] *= f;
    lds_fence();
  }
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const float p = __builtin_amdgcn_exp2f(s[hh] - st.m[hh]);
    st.l[hh] += p;
    st.c[hh] = fmaf(p, muv, st.c[hh]);
    const float x = p * sgx;
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    P[hh * 64 + lane] = hi;
    P[GM * 64 + hh * 64 + lane] = lo;
  }
  lds_fence();
}

// A operands of value step kk for tokens 32kk + 8G .. +7.  GM <= 8: one operand
// whose rows [0, GM) are the hi parts and rows [GM, 2 GM) the lo parts (P stores the
// lo rows right after the hi rows); GM = 16: hi and lo operands.  Other rows read
// the zero slot.
template <int GM>
__device__ __attribute__((always_inline)) inline void p_operands(const float* S, int kk, u32x4& ahi, u32x4& alo) {
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  const _Float16* P = (const _Float16*)S;
  constexpr int kZero = 2 * score_floats(GM);  // the zero slot, in halves
  if constexpr (GM <= 8) {
    ahi = *(const u32x4*)(P + (n < 2 * GM ? n * 64 + 32 * kk + 8 * G : kZero));
    alo = ahi;
  } else {
    ahi = *(const u32x4*)(P + (n < GM ? n * 64 + 32 * kk + 8 * G : kZero));
    alo = *(const u32x4*)(P + (n < GM ? GM * 64 + n * 64 + 32 * kk + 8 * G : kZero));
  }
}

// Quanta the last split of a (sequence, KV head) gives up to the others: half the
// quanta of an average split, at least 2 and at most 8 (the encode of an appended
// token and the later start of the split's query projection cost about 5-6 quanta of
// streaming, yet at 128K a cap of 8 measured ~0.6 us per step faster than 6; a split
// of few quanta cannot absorb it).
__host__ __device__ inline int split_slack(int nq, int ns) {
  const int e = nq / (2 * ns);
  return e < 2 ? 2 : (e > 8 ? 8 : e);
}

// Entry h of the first-workgroup table (16-bit entries, read through the 32-bit word
// that holds them: a scalar load).
__device__ inline int wg0_entry(const AttendArgs& a, int h) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(a.wg0)[h >> 1];
  return (int)((h & 1) ? w >> 16 : w & 0xFFFFu);
}

// The KV head of workgroup wr of a sequence's run: the last head whose first
// workgroup wg0[h] <= wr, i.e. the number of heads h >= 1 with wg0[h] <= wr (the
// table is non-decreasing).  The table's 32-bit words are scalar loads issued
// together and counted with scalar compares; a search through the 16-bit entries
// would take one dependent vector load per head.
__device__ inline int head_of_workgroup(const AttendArgs& a, int wr) {
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(a.wg0);
  const int nkv = a.n_kv_heads;
  int h = 0;
#pragma unroll
  for (int i = 0; i < kMaxKvHeads / 4; ++i) {
    const uint32_t w = w2[i];
    h += (2 * i >= 1 && 2 * i < nkv && (int)(w & 0xFFFFu) <= wr) ? 1 : 0;
    h += (2 * i + 1 < nkv && (int)(w >> 16) <= wr) ? 1 : 0;
  }
  if (nkv > kMaxKvHeads / 2) {
#pragma unroll
    for (int i = kMaxKvHeads / 4; i < kMaxKvHeads / 2; ++i) {
      const uint32_t w = w2[i];
      h += (2 * i < nkv && (int)(w & 0xFFFFu) <= wr) ? 1 : 0;
      h += (2 * i + 1 < nkv && (int)(w >> 16) <= wr) ? 1 : 0;
    }
  }
  return h;
}

// ----------------------------------------------------------------- kernel body
// One-dimensional grid of 256-thread workgroups; GM bounds the GQA group (g <= GM).
// Sequence b takes workgroups [b W, (b + 1) W) with W = wg_per_row: head h the
// heads.h[h].ns of them from wg0[h] on, one per split of its (b, h) unit, each
// split a quarter per wave; `run(ctx, state)` streams the wave's records and runs
// its online softmax.
// The four wave states are merged in LDS into one partial (m, l, o~[r_V]) per
// query head and split, and the last workgroup of the (sequence, KV head) to
// finish merges the splits and writes the output.
template <int GM, class Run>
__device__ __attribute__((always_inline)) inline void attend_body(const AttendArgs& a, Run&& run) {
  extern __shared__ float lds[];
#ifdef KVTC_STAMPS
  uint64_t* stamp = a.stamps ? a.stamps + (int64_t)blockIdx.x * kStampWords : nullptr;
  if (threadIdx.x == 0) {
    KVTC_STAMP(stamp, 0);
    if (stamp) {
      stamp[9] = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_REG_HW_ID, 32 bits
      stamp[10] = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11));  // HW_REG_XCC_ID
    }
  }
#else
  uint64_t* const stamp = nullptr;
#endif
  const int WA = tile_lds_words(a.kbuf_words, a.vbuf_words, a.nbuf, GM);
  const int b = (int)blockIdx.x / a.wg_per_row;
  const int wr = (int)blockIdx.x - b * a.wg_per_row;
  const int h = head_of_workgroup(a, wr);
  const int split = wr - wg0_entry(a, h);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the token loop scalar
  const HeadDesc hd = head_desc(a.heads, h);
  const int ns = hd.ns;
  const int g = __builtin_amdgcn_readfirstlane(a.group);
  const int rv = __builtin_amdgcn_readfirstlane(hd.rv);
  const int bv = __builtin_amdgcn_readfirstlane(hd.bv);
  const int NT = rv / 16;
  const int64_t bq0 = (int64_t)b * a.n_q_heads + (int64_t)h * g;
  if (tid == 0) KVTC_STAMP(stamp, 29);

  float* ml = lds;                                    // per wave: m[16] l[16] c[16]; then the flag word
  float* scores = lds + kCommonWords;                 // per wave: score_words(GM)
  float* areas = scores + kWaves * score_words(GM);   // per wave: WA words of record tiles
  float* wl = areas + wave * WA;

  WaveCtx c;
  // split x covers the 256-token quanta [q(x), q(x + 1)) of the nq in the context,
  // q(x) = min(nq, x ne / ns) with ne = nq + split_slack(nq, ns): the splits differ
  // by at most one quantum, so the XCDs (which take the splits round-robin) stream
  // equal shares, and the last split (which holds the newest token, the one a fused
  // append encodes first) is split_slack quanta lighter, about the time that encode
  // and the later start of its query projection take (measured with phase stamps
  // at 128K: 9.5 us of encode and a 2 us slower projection, against ~2 us per
  // quantum of a 21-quantum split).  Both entry points use the same splits, so
  // appending in the same launch leaves the result bit for bit unchanged.
  // this sequence's context: n_tokens, or its own length (clamped to [0, n_tokens])
  int n_tok = (int)a.n_tokens;
  if (a.lengths) {
    const int lb = a.lengths[b];
    n_tok = lb < 0 ? 0 : (lb < n_tok ? lb : n_tok);
  }
  const int nq = (n_tok + kSplitQuantum - 1) / kSplitQuantum;
  const int ne = nq + split_slack(nq, ns);
  const int q0 = min(nq, (int)(((int64_t)split * ne) / ns));
  const int q1 = min(nq, (int)(((int64_t)split * ne + ne) / ns));
  const int s_begin = q0 * kSplitQuantum;
  const int s_end = q1 * kSplitQuantum < n_tok ? q1 * kSplitQuantum : n_tok;
  const int wq = (q1 - q0) * (kSplitQuantum / kWaves);
  c.t_begin = s_begin + wave * wq;
  c.t_end = c.t_begin + wq;
  if (c.t_end > n_tok) c.t_end = n_tok;
  if (tid == 0) KVTC_STAMP(stamp, 30);
  c.split_begin = s_begin;
  c.wave_tokens = wq;
  c.n_tok = n_tok;
  c.wave_area = WA;
  c.extra = areas + kWaves * WA;
  const int wk = hd.wk, wv = hd.wv;
  // buffer resources over the sequence's records (contiguous) or the head's pool (paged)
  const bool paged = a.pg.bt != nullptr;
  const int64_t rbase = paged ? 0 : (int64_t)b * a.capacity;
  const uint32_t nrec = paged ? (uint32_t)(a.pg.pool_pages * a.pg.page) : (uint32_t)a.capacity;
  const uint32_t* kreg = a.cache_k + hd.base_k + rbase * wk;
  const uint32_t* vreg = a.cache_v + hd.base_v + rbase * wv;
  c.rk_ = make_rsrc(kreg, nrec * 4u * wk);
  c.rv_ = make_rsrc(vreg, nrec * 4u * wv);
  c.bt_row = paged ? a.pg.bt + (int64_t)b * a.pg.pages_per_seq : nullptr;
  c.page = a.pg.page;
  c.pool_recs = nrec;
  c.pool_pages = a.pg.pool_pages;
  c.kbuf = a.kbuf_words;
  c.vbuf = a.vbuf_words;
  c.nbuf = a.nbuf;
  c.ktile = (uint32_t*)wl;
  c.vtile = c.ktile + c.nbuf * c.kbuf;
  c.S = scores + wave * score_words(GM);
  c.stage = scores;
  c.stats = ml + kWaves * 48 + 4;
  c.g = g;
  c.h = h;
  c.b = b;
  c.unit = (int64_t)b * a.n_kv_heads + h;
  c.stamp = stamp;
  c.cbk = c.cbv = nullptr;
  if (a.cb_words > 0 && !a.rope) {  // vector-quantized records: the head's codebooks after the tile areas,
                         // one row of 2^b entries per pair at the padded strides of the phases
    uint32_t* cbl = (uint32_t*)(areas + kWaves * WA);
    const int ek = code_bits(hd.bk), ev = code_bits(hd.bv);
    const int nk = codebook_words(hd.rk, hd.bk), nv = codebook_words(hd.rv, hd.bv);
    const int sk = vq_kstride(hd.bk, hd.rk), sv = vq_vstride(hd.bv);
    const int lk = is_vq(hd.bk) ? (hd.rk / 2) * sk : 0;
    for (int i = tid; i < nk; i += 256) cbl[(i >> ek) * sk + (i & ((1 << ek) - 1))] = a.cb_k[hd.sk + i];
    for (int i = tid; i < nv; i += 256) cbl[lk + (i >> ev) * sv + (i & ((1 << ev) - 1))] = a.cb_v[hd.sv + i];
    c.cbk = cbl;
    c.cbv = cbl + lk;  // read after the barriers of the query projection
  }

  // append fused with attention: the workgroup whose split holds the new token
  // encodes its key and value (waves 0-1 and 2-3) before any of its tiles stream in
  const int64_t append_rec = a.append_pos >= s_begin && a.append_pos < s_end
                                 ? record_index(a.pg, a.capacity, b, a.append_pos) : -1;
  if (append_rec >= 0) {
    EncodeScratch* scr = (EncodeScratch*)scores;  // score and tile areas are not in use yet
    const int tensor = tid >> 7, t = tid & 127;
    const int r = tensor ? hd.rv : hd.rk, bits = tensor ? hd.bv : hd.bk, W = tensor ? hd.wv : hd.wk;
    const int hdr = tensor ? hd.hv : hd.hk;
    const uint32_t sw = tensor ? hd.sv : hd.sk;
    const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
    const uint32_t* cbt = is_vq(bits) ? (tensor ? a.cb_v : a.cb_k) + sw : nullptr;
    const int64_t xo = ((int64_t)b * a.n_kv_heads + h) * kHeadDim;
    // the fused entry point hands writable caches (kv_append_attend_decode)
    uint32_t* rec = const_cast<uint32_t*>(tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k) + append_rec * W;
    auto sync = [] { __syncthreads(); };
    if (a.append_dtype == 0)
      encode_token_128((const float*)(tensor ? a.v1 : a.k1) + xo, P, r, bits, hdr, sw, cbt, rec, scr[tensor], t, sync);
    else
      encode_token_128((const _Float16*)(tensor ? a.v1 : a.k1) + xo, P, r, bits, hdr, sw, cbt, rec, scr[tensor], t,
                       sync);
    // the records are in L2 before any tile copy (the builtin, unlike an asm wait, also
    // tells the compiler that no store of the encoder is outstanding any more)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) KVTC_STAMP(stamp, 11);
  }

  if (tid == 0) KVTC_STAMP(stamp, 31);
  WaveState<GM> st;
  run(c, st);
  wait_tiles();
  if (lane == 0) KVTC_STAMP(stamp, 2 + wave);
  // The tile loop ends at issue priority 0 (progress_priority); the epilogue and the
  // split merge are short and gate the unit's output (and, for the last workgroups, the
  // launch), so they take the highest priority over the streaming waves of the CU.
  __builtin_amdgcn_s_setprio(3);

  // ---- wave partial: m, l, sum of p*min (per head), o~[head][j] in natural code order
  const int n = lane & 15, G = lane >> 4;
  float* mlw = ml + wave * 48;
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const float ls = wave_sum_uniform(st.l[hh]);
    const float cs = wave_sum_uniform(st.c[hh]);
    if (lane == 0 && hh < g) {
      mlw[hh] = st.m[hh];
      mlw[16 + hh] = ls;
      mlw[32 + hh] = cs;
    }
  }
  lds_fence();
  // accumulator row 4G + e: head (4G + e) mod GM, the lo part of the packed value
  // operand for rows >= GM (GM <= 8); the sum p*min joins the hi row
  constexpr int kRows = GM <= 8 ? 2 * GM : GM;
  if (4 * G < kRows) {
    // the sums p * min of this lane group's heads (4G + e) mod GM, read once: read inside
    // the store loop, each store would wait for a read behind the previous store
    const f32x4 cs4 = *(const f32x4*)(mlw + 32 + ((4 * G) & (GM - 1)));
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      if (nt < NT) {
        const float f = ldexpf(1.0f, (is_vq(bv) ? 0 : 24) - kPScale - v_shift(bv, nt));  // VQ: normal operands
        const int j = n * NT + nt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * G + e, hh = row & (GM - 1);
          if (hh < g) wl[row * rv + j] = fmaf(st.acc2[nt][e], f, row < GM ? cs4[e] : 0.0f);
        }
      }
    }
  }

  if (lane == 0) KVTC_STAMP(stamp, 16 + wave);
  // this thread's half row of P_V for the back-projection of the workgroup's partial,
  // in flight during the wave merge (issued once the value accumulators are free):
  // segment [bhalf jh, bhalf jh + jh) of row bi, jh = r_V / 2, in float4 steps;
  // steps past the segment re-read its first one and meet zeros in the staged
  // partial, so that no load or product is conditional (a data-dependent branch
  // here costs a full memory wait per step)
  const int bi = tid >> 1, bhalf = tid & 1, jh = rv / 2;
  const float* prow = a.basis_v + hd.boff_v + (int64_t)bi * rv + bhalf * jh;
  float4 pv[kMaxRank / 8];
#pragma unroll
  for (int k = 0; k < kMaxRank / 8; ++k) pv[k] = *(const float4*)(prow + (4 * k < jh ? 4 * k : 0));
  if (lane == 0) KVTC_STAMP(stamp, 20 + wave);
  __syncthreads();
  if (tid == 0) KVTC_STAMP(stamp, 12);

  // ---- merge the four wave partials into one partial o~ per query head, staged
  // in the score area (free after the token loop) as ot[head][half][64]: half h of
  // head row holds o~[bhalf jh .. bhalf jh + jh) and zeros after it, rows >= g are
  // zero.  Waves without tokens carry m = -1e30, l = 0 and a zero partial, so
  // their weight is 0.  Then the back-projection P_V o~.
  float* part0 = a.part + (bq0 * a.n_splits + split) * (int64_t)kPartStride;
  float* ot = scores;  // [GM][2][64]
#pragma unroll
  for (int i = 0; i < GM / 2; ++i) {
    const int o = tid + 256 * i;
    const int hh = o >> 7, half = (o >> 6) & 1, m = o & 63;
    const bool on = hh < g && m < jh;
    const int hc = hh < g ? hh : 0, j = half * jh + (m < jh ? m : 0);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[w * 48 + hc]);
    float acc = 0.0f, lacc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wgt = exp2f(ml[w * 48 + hc] - M);
      const float* aw = areas + w * WA + hc * rv + j;
      acc = fmaf(wgt, GM <= 8 ? aw[0] + aw[GM * rv] : aw[0], acc);
      lacc = fmaf(wgt, ml[w * 48 + 16 + hc], lacc);
    }
    ot[o] = on ? acc : 0.0f;
    if (on && o == hh * 128) {
      float* ph = part0 + (int64_t)hh * a.n_splits * kPartStride;
      part_store(ph + kPartM, M);
      part_store(ph + kPartL, lacc);
      part_store_u32(ph + kPartTag, a.nonce);
    }
  }
  __syncthreads();
  if (tid == 0) KVTC_STAMP(stamp, 13);
  {
    float accb[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) accb[hh] = 0.0f;
    // one step per float4 of the row segment: the staged reads of a step are issued
    // together (the uniform bound keeps the scheduler from hoisting all of them,
    // which would not fit the register budget)
#pragma unroll
    for (int k = 0; k < kMaxRank / 8; ++k) {
      if (4 * k < jh) {
        f32x4 o4[GM];
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) o4[hh] = *(const f32x4*)(ot + hh * 128 + bhalf * 64 + 4 * k);
#pragma unroll
        for (int hh = 0; hh < GM; ++hh)
          accb[hh] = fmaf(pv[k].x, o4[hh][0], fmaf(pv[k].y, o4[hh][1], fmaf(pv[k].z, o4[hh][2], fmaf(pv[k].w, o4[hh][3], accb[hh]))));
      }
    }
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      const float v = accb[hh] + __shfl_xor(accb[hh], 1);
      if (hh < g && bhalf == 0) part_store(part0 + (int64_t)hh * a.n_splits * kPartStride + bi, v);
    }
  }
  if (tid == 0) KVTC_STAMP(stamp, 14);

  // ---- arrival: the last workgroup of this (sequence, KV head) merges all splits.
  // A counter that was not zero on entry makes later arrivals (count past ns) merge
  // too; the partial tags keep any of those merges from folding a stale partial.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores have completed
  __syncthreads();
  if (tid == 0) KVTC_STAMP(stamp, 6);
  uint32_t* flag = (uint32_t*)(ml + kWaves * 48);
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.cnt + c.unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t arrived = (uint64_t)prev + 1u;
    *flag = arrived == (uint64_t)ns ? 1u : (arrived > (uint64_t)ns ? 2u : 0u);
  }
  __syncthreads();
  if (tid == 0) KVTC_STAMP(stamp, 7);
  const uint32_t fl = *flag;
  if (fl == 0u) return;
  merge_splits(a, h, b, fl == 1u);
  if (tid == 0) KVTC_STAMP(stamp, 8);
}

}  // namespace kvtc
