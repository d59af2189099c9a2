// Prefill encoder for gfx950: the (tokens x 128) by (128 x r) basis contraction
// of every (sequence, KV head, tensor) on the matrix cores, with the quantizer's
// rounding decisions kept exact.
//
// KV-COBRA project page, "How KV-COBRA Works" (Inference): each key (and value)
// is rotated and truncated with its head's basis and quantized with its head's
// b-bit quantizer; at prefill that projection is one dense contraction per head.
//
// Arithmetic.  Each basis element (fp32), scaled by 2^8, is split into two fp16
// parts, 2^8 P = Ph + Pl + e with |e| <= 2^-22 |2^8 P| + 2^-25, and fp32 inputs the
// same way (fp16 inputs are exact operands); the sums are scaled back by 2^-8,
// exactly.  v_mfma_f32_16x16x32_f16 on gfx950 does not return the exact sum of its
// 32 products and accumulator rounded once: probed on random operands (the matrix-
// core probe and its tests), about half of its results differ from that, and with
// normal fp16 operands of the encoder's kind (basis parts, Gaussian inputs with
// outlier channels and subnormal inputs, accumulators of the size of the partial
// sums) its error reaches 3.5u (|C| + sum |p|) (u = 2^-24).  The encoder takes
// k = 4 per instruction: err <= 4u (|C| + sum |p|).  Over the 8 chained
// instructions of a coordinate, with |C| at most the partial sum of the product
// magnitudes so far and S_j = sum_i |x_i P_ij| <= ||x||_2 ||P_j||_2 <= ||x||_2 n_P
// (n_P: the largest column norm of the basis, formed while it is staged, slightly
// rounded up; 1 for an orthonormal basis, more or less for a non-orthogonal key
// transform), the error is at most 8k u S_j = 32u S_j, and the split remainders add
// 4u S_j (the absolute part, 2^-33 ||x||_1 n_P, is negligible).  The encoder uses
//     E = 48u ||x||_2 n_P
// for fp16 inputs, 1.33 times that bound (fp32 inputs: three products per term, 24
// instructions, 24k u + 8u, and the absolute split error of inputs below the fp16
// normal range: E = (144u ||x||_2 + 2^-21) n_P; they must lie inside the fp16
// range, |x| < 65504).  The bound rests on the probed factor k, not on a documented
// one; the probe's tests check k on every run of the GPU suite.  The header (fp16 min
// and step) and the codes are monotone functions of the coordinates, so a
// decision that takes the same value at c~ - E and c~ + E is the exact decision.
// The others are recomputed from the float64 projection in the fixed summation
// order every encode path uses (four groups of 32 rows, then the group sums in
// order):
//   * a token whose fp16 min or step could round either way gets the exact
//     values of its extreme candidates (c~ within 2E of the approximate min or
//     max), which contain the exact extremes, and its header from them;
//   * a coordinate whose code could round either way gets its exact value.
// The records are then the float64 encoder's records, bit for bit.
#include "encode_core.h"
#include "kvtc_common.h"
#include "kvtc_launch.h"

namespace kvtc {
namespace {

typedef _Float16 enc_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 enc_half2 __attribute__((ext_vector_type(2)));
typedef float enc_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t enc_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kEncWaves = 4;

__device__ inline enc_f32x4 mma(enc_half8 a, enc_u32x4 b, enc_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(enc_half8, b), c, 0, 0, 0);
}

// Eight consecutive input elements as floats.
__device__ inline void load8(const _Float16* p, float (&f)[8]) {
  const enc_half8 h = *(const enc_half8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ inline void load8(const float* p, float (&f)[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ inline uint32_t h16_bits(float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); }

// Four codes (bytes of v, codes < 16) as one 16-bit field, and (codes < 4) as one byte.
__device__ inline uint32_t compact4(uint32_t v) {
  v = (v | (v >> 4)) & 0x00FF00FFu;
  return (v | (v >> 8)) & 0xFFFFu;
}
__device__ inline uint32_t compact2(uint32_t v) {
  v = (v | (v >> 6)) & 0x000F000Fu;
  return (v | (v >> 12)) & 0xFFu;
}

// LDS ordering among the lanes of one wave.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum of v over the wave's lanes; the sum over all lanes in total.
__device__ inline int wave_prefix(int v, int lane, int& total) {
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  total = __shfl(x, 63);
  return x - v;
}

// A coordinate to recompute: token 16nt + n of the wave, coordinate 16(s/4) + 4G + s%4.
__device__ inline uint32_t item_code(int nt, int n, int G, int s) {
  return ((uint32_t)(16 * nt + n) << 8) | (uint32_t)(16 * (s >> 2) + 4 * G + (s & 3));
}

constexpr int kRepairList = 64;  // items one wave recomputes per round

// Exact values of the `cnt` listed coordinates (cnt <= kRepairList), four lanes per
// item, lane 4i + q summing rows 32q .. 32q+31 of item i in order; the group sums
// are added in the fixed order, so each value is the float64 encoder's.  A lane
// issues all 64 loads of its row group (32 inputs, 32 basis elements) before the
// first product, so a round costs one memory latency.  P is the basis in memory or
// its float32 copy in LDS.
template <typename T>
__device__ inline void coop_exact(const uint32_t* items, double* res, int cnt, const T* xu, int64_t wtok0,
                                  const float* P, int R, int lane) {
  wave_sync();
  const int q = lane & 3, l0 = lane & ~3;
#pragma unroll 1
  for (int base = 0; base < cnt; base += 16) {
    const int it = base + (lane >> 2);
    double g = 0.0;
    if (it < cnt) {
      const uint32_t e = items[it];
      const T* row = xu + (wtok0 + (int64_t)(e >> 8)) * kHeadDim + 32 * q;
      const float* pc = P + 32 * q * R + (int)(e & 255u);
      constexpr int kVec = 16 / sizeof(T);  // inputs per 16-byte load, kept packed
      typedef T xvec __attribute__((ext_vector_type(kVec)));
      xvec xv[32 / kVec];
      float pv[32];
#pragma unroll
      for (int c = 0; c < 32 / kVec; ++c) xv[c] = *(const xvec*)(row + kVec * c);
#pragma unroll
      for (int i = 0; i < 32; ++i) pv[i] = pc[i * R];
#pragma unroll
      for (int i = 0; i < 32; ++i) g = fma((double)xv[i / kVec][i % kVec], (double)pv[i], g);
    }
    const double g0 = __shfl(g, l0), g1 = __shfl(g, l0 + 1), g2 = __shfl(g, l0 + 2), g3 = __shfl(g, l0 + 3);
    if (q == 0 && it < cnt) res[it] = ((g0 + g1) + g2) + g3;
  }
  wave_sync();
}

// Dynamic LDS: the basis as fp16 hi/lo A operands (R x 128 x 4 bytes); for R <= 32
// also the basis in float32 (the exact recomputations read it there; for larger R
// it would cost a resident workgroup per CU, and they read it from memory); then
// per wave one 16-token block: the records being assembled ([16][W] words, header
// first) for b = 2, 4, 8, or the codes ([16][R] bytes) and headers for other b;
// and one round of coordinates to recompute with their exact values.
__host__ __device__ constexpr bool enc_p32(int R) { return R <= 32; }
__host__ __device__ constexpr int enc_base_bytes(int R) { return R * kHeadDim * (enc_p32(R) ? 8 : 4); }
__host__ __device__ constexpr int enc_wave_bytes(int R) { return 16 * R + 128 + kRepairList * 12; }
__host__ __device__ constexpr int enc_lds_bytes(int R) { return enc_base_bytes(R) + kEncWaves * enc_wave_bytes(R); }

// Grid: x = groups of `tiles_per_wg` token tiles, y = the (head, tensor) units of
// rank R (keys of the heads in mask_k, then values of the heads in mask_v), z =
// sequence.  Each wave projects 16*NT tokens per tile: A = P^T (hi and lo parts)
// from LDS, B = the tokens' inputs straight from HBM, one 16 x 16
// coordinate-by-token accumulator per (coordinate block, token block).  Lane
// (n, G) = (lane % 16, lane / 16) ends with coordinates 16mb + 4G + i of token n.
template <typename T, int R, int NT, bool PF, int OCC>
__global__ __launch_bounds__(256, OCC) void encode_mfma_kernel(EncodeArgs a, uint64_t mask_k, uint64_t mask_v,
                                                               int tiles_per_wg) {
  constexpr int MB = R / 16;
  constexpr int NS = MB * 4;  // coordinates per lane and token
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int kWaveTok = 16 * NT;
  constexpr int kTileTok = kEncWaves * kWaveTok;
  extern __shared__ float enc_lds[];
  uint8_t* ab = (uint8_t*)enc_lds;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* wb = ab + enc_base_bytes(R) + wave * enc_wave_bytes(R);
  uint32_t* recw = (uint32_t*)wb;                  // b = 2, 4, 8: [16][W] words
  uint32_t* hdrw = (uint32_t*)(wb + 16 * R + 64);  // other b: header words
  double* res = (double*)(wb + 16 * R + 128);       // exact values of the listed coordinates
  uint32_t* items = (uint32_t*)(res + kRepairList);

  // the unit: blockIdx.y-th set bit of mask_k, then of mask_v
  const int nk = __popcll(mask_k);
  int idx = blockIdx.y;
  const int tensor = idx >= nk;
  const uint64_t mask = tensor ? mask_v : mask_k;
  if (tensor) idx -= nk;
  int h = 0;
  for (; h < kMaxKvHeads - 1; ++h) {  // the grid has one y per set bit, so the search ends on one
    if ((mask >> h) & 1ull) {
      if (idx == 0) break;
      --idx;
    }
  }
  h = __builtin_amdgcn_readfirstlane(h);
  const int b = blockIdx.z;
  const HeadDesc& hd = a.heads.h[h];
  const int bits = tensor ? hd.bv : hd.bk;
  const int W = tensor ? hd.wv : hd.wk;             // words of a stored record
  const int hdr = tensor ? hd.hv : hd.hk;           // 0: header-free, the head's fixed min and step
  const uint32_t sw = tensor ? hd.sv : hd.sk;
  const int WI = W + 1 - hdr;                       // words of a record assembled in LDS (header slot first)
  const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
  const T* xu = (const T*)(tensor ? a.v : a.k) + ((int64_t)b * a.n_kv_heads + h) * a.n_tokens * kHeadDim;
  uint32_t* region = tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k;  // the head's records

  // stage the basis as A operands: for (mb, ks, lane) the eight rows 32ks + 8G ..
  // of column 16mb + m, hi parts then (64 lanes later) lo parts; the basis is scaled
  // by 2^8 (undone exactly on the sums) so that the lo parts of its elements stay in
  // the fp16 normal range down to |P| = 2^-11
  __shared__ float colsq[kMaxRank];  // squared column norms of the basis (times 2^16)
  if (tid < R) colsq[tid] = 0.0f;
  __syncthreads();
  for (int q = tid; q < R * 16; q += 256) {
    const int ln = q & 63, ks = (q >> 6) & 3, mb = q >> 8;
    const int k0 = 32 * ks + 8 * (ln >> 4), j = 16 * mb + (ln & 15);
    enc_half8 hi, lo;
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = P[(k0 + i) * R + j] * 0x1p8f;
      sq = fmaf(p, p, sq);
      hi[i] = (_Float16)p;
      lo[i] = (_Float16)(p - (float)hi[i]);
    }
    atomicAdd(&colsq[j], sq);
    uint8_t* dst = ab + (((mb * 4 + ks) * 2 * 64 + ln) << 4);
    *(enc_half8*)dst = hi;
    *(enc_half8*)(dst + 1024) = lo;
  }
  float* p32 = (float*)(ab + R * kHeadDim * 4);
  if constexpr (enc_p32(R))
    for (int q = tid; q < R * kHeadDim; q += 256) p32[q] = P[q];
  const float* Px = enc_p32(R) ? (const float*)p32 : P;  // the basis the recomputations read
  __syncthreads();

  // n_P, the largest column norm: the float32 sums of squares, rounded up by far more than
  // their rounding error
  float pn2 = 0.0f;
  for (int j = lane; j < R; j += 64) pn2 = fmaxf(pn2, colsq[j]);
  for (int o = 32; o > 0; o >>= 1) pn2 = fmaxf(pn2, __shfl_xor(pn2, o));
  const float pnorm = __builtin_sqrtf(pn2) * 0x1p-8f * 1.0001f;
  const float top = (float)((1 << bits) - 1);
  const float kinv = 1.0f / top;
  const bool pow2 = (bits & (bits - 1)) == 0;
  const uint32_t wmagic = (uint32_t)((0x100000000ull + W - 1) / W);
  const int64_t n_tiles = (a.n_tokens + kTileTok - 1) / kTileTok;
  // B operands: lane (n, G) holds dims 32ks + 8G .. +7 of token 16nt + n.  fp16
  // inputs are the operands as loaded; the next tile's are loaded while this
  // tile's coordinates are quantized.
  enc_u32x4 bh[4][NT], bl[4][NT];
  auto load_f16 = [&](int64_t tile_) {
    const int64_t t0 = tile_ * kTileTok + wave * kWaveTok;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t tok = t0 + 16 * nt + n;
      const T* row = xu + tok * kHeadDim + 8 * G;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        enc_u32x4 v = {0u, 0u, 0u, 0u};
        if (tok < a.n_tokens) v = *(const enc_u32x4*)(row + 32 * ks);
        bh[ks][nt] = v;
      }
    }
  };
  if constexpr (!kF32 && PF) {
    if ((int64_t)blockIdx.x * tiles_per_wg < n_tiles) load_f16((int64_t)blockIdx.x * tiles_per_wg);
  }
#pragma unroll 1
  for (int it = 0; it < tiles_per_wg; ++it) {
    const int64_t tile = (int64_t)blockIdx.x * tiles_per_wg + it;
    if (tile >= n_tiles) break;
    const int64_t wtok0 = tile * kTileTok + wave * kWaveTok;
    if constexpr (!kF32 && !PF) load_f16(tile);

    float ss[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ss[nt] = 0.f;
    if constexpr (kF32) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t tok = wtok0 + 16 * nt + n;
        const T* row = xu + tok * kHeadDim + 8 * G;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (tok < a.n_tokens) load8(row + 32 * ks, f);
          enc_half8 hi, lo;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            hi[i] = (_Float16)f[i];
            lo[i] = (_Float16)(f[i] - (float)hi[i]);
            ss[nt] = fmaf(f[i], f[i], ss[nt]);
          }
          bh[ks][nt] = __builtin_bit_cast(enc_u32x4, hi);
          bl[ks][nt] = __builtin_bit_cast(enc_u32x4, lo);
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const enc_half2 v = __builtin_bit_cast(enc_half2, bh[ks][nt][p]);
            ss[nt] = __builtin_amdgcn_fdot2(v, v, ss[nt], false);
          }
    }

    // ---- contraction: acc[mb][nt] = P^T(block mb) x X^T(block nt)
    enc_f32x4 acc[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = enc_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint8_t* src = ab + (((mb * 4 + ks) * 2 * 64 + lane) << 4);
        const enc_half8 ah = *(const enc_half8*)src, al = *(const enc_half8*)(src + 1024);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mb][nt] = mma(ah, bh[ks][nt], acc[mb][nt]);
          acc[mb][nt] = mma(al, bh[ks][nt], acc[mb][nt]);
          if constexpr (kF32) acc[mb][nt] = mma(ah, bl[ks][nt], acc[mb][nt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keeps the operand reads of later row blocks from piling up
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mb][nt] *= 0x1p-8f;  // the basis scale, exactly
    if constexpr (!kF32 && PF) {
      if (it + 1 < tiles_per_wg && tile + 1 < n_tiles) load_f16(tile + 1);
    }

    // ---- headers of the wave's 16*NT tokens from the approximate extremes, if every
    // value within E gives the same fp16 min and step (fp32 interval ends, hardware
    // round-to-nearest-even: the interval is many fp32 ulps wide, so it settles the
    // float64 decision too); the others from the exact values of their candidates
    float Ev[NT];
    uint32_t w0[NT], cand[NT];
    bool hbad[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bool valid = wtok0 + 16 * nt + n < a.n_tokens;
      float s2 = ss[nt];
      s2 += __shfl_xor(s2, 16);
      s2 += __shfl_xor(s2, 32);
      float mn = acc[0][nt][0], mx = acc[0][nt][0];
#pragma unroll
      for (int s = 1; s < NS; ++s) {
        mn = fminf(mn, acc[s >> 2][nt][s & 3]);
        mx = fmaxf(mx, acc[s >> 2][nt][s & 3]);
      }
      mn = fminf(mn, __shfl_xor(mn, 16));
      mn = fminf(mn, __shfl_xor(mn, 32));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // error bound of the coordinates (see the top of the file); an fp32 input below
      // the fp16 normal range keeps an absolute split error of up to 2^-25 per
      // element, at most 2^-25 * ||P_j||_1 <= 2^-21.5 ||P_j||_2 per coordinate
      const float E = (kF32 ? 0x1.2p-17f * __builtin_sqrtf(s2) + 0x1p-21f : 0x1.8p-19f * __builtin_sqrtf(s2)) * pnorm;
      Ev[nt] = E;
      const uint32_t m_lo = h16_bits(mn - E), m_hi = h16_bits(mn + E);
      const float muf0 = f16_bits_to_f32(m_lo);
      const uint32_t s_lo = h16_bits(fmaxf(mx - E - muf0, 0.f) * kinv);
      const uint32_t s_hi = h16_bits(fmaxf(mx + E - muf0, 0.f) * kinv);
      w0[nt] = hdr ? (m_lo | (s_lo << 16)) : sw;
      hbad[nt] = hdr && valid && (m_lo != m_hi || s_lo != s_hi);
      cand[nt] = 0u;
      if (hbad[nt]) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const float c = acc[s >> 2][nt][s & 3];
          if (c <= mn + 2.f * E || c >= mx - 2.f * E) cand[nt] |= 1u << s;
        }
      }
    }
    {
      int mine = 0;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mine += __popc(cand[nt]);
      if (__ballot(mine != 0)) {
        int total;
        const int off = wave_prefix(mine, lane, total);
        double emin[NT], emax[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          emin[nt] = __builtin_inf();
          emax[nt] = -__builtin_inf();
        }
#pragma unroll 1
        for (int base = 0; base < total; base += kRepairList) {  // rounds of kRepairList items
          const int cnt = total - base < kRepairList ? total - base : kRepairList;
          int k = off;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            for (uint32_t m = cand[nt]; m; m &= m - 1u, ++k)
              if (k >= base && k < base + cnt) items[k - base] = item_code(nt, n, G, __builtin_ctz(m));
          coop_exact(items, res, cnt, xu, wtok0, Px, R, lane);
          k = off;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            for (uint32_t m = cand[nt]; m; m &= m - 1u, ++k)
              if (k >= base && k < base + cnt) {
                emin[nt] = fmin(emin[nt], res[k - base]);
                emax[nt] = fmax(emax[nt], res[k - base]);
              }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          double lo = emin[nt], hi = emax[nt];
          lo = fmin(lo, __shfl_xor(lo, 16));
          lo = fmin(lo, __shfl_xor(lo, 32));
          hi = fmax(hi, __shfl_xor(hi, 16));
          hi = fmax(hi, __shfl_xor(hi, 32));
          if (hbad[nt]) w0[nt] = quant_header(lo, hi, bits).word0;
        }
        wave_sync();
      }
    }

    // ---- per 16-token block: codes, exact codes near rounding boundaries, store
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t tok = wtok0 + 16 * nt + n;
      const bool valid = tok < a.n_tokens;
      // q = (c - min) / step + 1/2, code = floor(q) clamped, unless q is within tol
      // of an integer (tol: the coordinate bound E, and 4u (2^b) for the fp32 steps)
      const float muf = f16_bits_to_f32(w0[nt] & 0xFFFFu), sgf = f16_bits_to_f32(w0[nt] >> 16);
      const bool sig_pos = valid && sgf > 0.f;
      const float inv = sgf > 0.f ? 1.0f / sgf : 0.f;
      const float tol = Ev[nt] * inv * 1.0001f + (top + 1.f) * 0x1p-22f;
      uint32_t fl = 0u;
      uint32_t* rec = recw + n * WI;
      if (G == 0) {
        if (pow2) rec[0] = w0[nt];
        else hdrw[n] = w0[nt];
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        uint32_t v = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float q = fmaf(acc[mb][nt][i] - muf, inv, 0.5f);
          const float fr = __builtin_amdgcn_fractf(q);
          if (__builtin_fabsf(fr - 0.5f) > 0.5f - tol) fl |= 1u << (4 * mb + i);
          v = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(q - fr, 0.f, top), i, v);
        }
        const int j0 = 16 * mb + 4 * G;  // first of the four coordinates
        if (bits == 8) rec[1 + (j0 >> 2)] = v;
        else if (bits == 4) ((uint16_t*)(rec + 1))[j0 >> 2] = (uint16_t)compact4(v);
        else if (bits == 2) ((uint8_t*)(rec + 1))[j0 >> 2] = (uint8_t)compact2(v);
        else *(uint32_t*)(wb + n * R + j0) = v;
      }
      if (!sig_pos) fl = 0u;
      if (__ballot(fl != 0u)) {  // exact codes of the flagged coordinates, in rounds
        int total;
        const int off = wave_prefix(__popc(fl), lane, total);
        const double mu = (double)muf, sg = (double)sgf;
#pragma unroll 1
        for (int base = 0; base < total; base += kRepairList) {
          const int cnt = total - base < kRepairList ? total - base : kRepairList;
          int k = off;
          for (uint32_t m = fl; m; m &= m - 1u, ++k)
            if (k >= base && k < base + cnt) items[k - base] = item_code(nt, n, G, __builtin_ctz(m));
          coop_exact(items, res, cnt, xu, wtok0, Px, R, lane);
          k = off;
          for (uint32_t m = fl; m; m &= m - 1u, ++k) {
            if (k < base || k >= base + cnt) continue;
            const int s = __builtin_ctz(m);
            const int j = 16 * (s >> 2) + 4 * G + (s & 3);
            const uint32_t code = quant_code(res[k - base], mu, sg, bits);
            if (pow2) {  // codes of other lanes share the word: atomic field update
              const int bit = j * bits;
              const uint32_t sh = bit & 31, fm = ((1u << bits) - 1u) << sh;
              atomicAnd(rec + 1 + (bit >> 5), ~fm);
              atomicOr(rec + 1 + (bit >> 5), code << sh);
            } else {
              wb[n * R + j] = (uint8_t)code;
            }
          }
        }
      }
      wave_sync();

      // store the block's records, each at its record index (consecutive for
      // contiguous caches, through the block table for paged ones); f / W as a
      // multiply-high by ceil(2^32 / W), exact for f < 2^16 (a one-word header-free
      // record, whose magic would not fit 32 bits, is its own quotient)
      const int64_t btok0 = wtok0 + 16 * nt;
      for (int f = lane; f < 16 * W; f += 64) {
        const int tn = W == 1 ? f : (int)__umulhi((uint32_t)f, wmagic), wi = f - tn * W + 1 - hdr;
        const int64_t ri = btok0 + tn < a.n_tokens ? record_index(a.pg, a.capacity, b, a.pos0 + btok0 + tn) : -1;
        if (ri >= 0) {
          uint32_t word;
          if (pow2) word = recw[tn * WI + wi];
          else word = wi == 0 ? hdrw[tn] : pack_word(wb + tn * R, R, bits, wi - 1);
          region[ri * W + (f - tn * W)] = word;
        }
      }
      wave_sync();
    }
  }
}

// Launch shapes per (input type, rank), from measurements of the 128K-context
// allocations: 16-token blocks per wave (NT), whether the next tile's inputs are
// loaded during quantization (PF), and workgroups per CU (OCC, bounds registers).
template <typename T, int R>
struct EncShape {
  static constexpr bool kF32 = sizeof(T) == 4;
  static constexpr int NT = kF32 ? (R == 128 ? 1 : 2) : (R == 16 ? 4 : 2);
  static constexpr bool PF = !kF32 && R == 32;
  static constexpr int OCC = (!kF32 && R <= 64) ? 3 : 2;
};

template <typename T, int R>
hipError_t launch_rank(const EncodeArgs& a, uint64_t mask_k, uint64_t mask_v, hipStream_t s) {
  using S = EncShape<T, R>;
  const int units = __builtin_popcountll(mask_k) + __builtin_popcountll(mask_v);
  if (units == 0) return hipSuccess;
  constexpr int kTileTok = kEncWaves * 16 * S::NT;
  const int64_t n_tiles = (a.n_tokens + kTileTok - 1) / kTileTok;
  // Tiles per workgroup: each workgroup stages the basis once for its tiles (for r =
  // 128 that staging reads as many bytes as two tiles of fp16 inputs), so a chunk
  // that fits the resident workgroups in one round gives each of them an equal share
  // (one round of resident workgroups, each staging once); larger chunks run about
  // 2048 workgroups or more, up to 8 tiles each.
  const int64_t per_tile_row = (int64_t)units * a.batch;
  const int64_t total = n_tiles * per_tile_row;
  const int64_t lds_per_cu = (160 * 1024) / enc_lds_bytes(R);
  const int64_t resident = 256 * (lds_per_cu < S::OCC ? lds_per_cu : S::OCC);
  int64_t tpw = total / 2048;
  if (tpw < 1) tpw = (total + resident - 1) / resident;
  tpw = tpw < 1 ? 1 : (tpw > 8 ? 8 : tpw);
  const dim3 grid((unsigned)((n_tiles + tpw - 1) / tpw), (unsigned)units, (unsigned)a.batch);
  hipLaunchKernelGGL((encode_mfma_kernel<T, R, S::NT, S::PF, S::OCC>), grid, dim3(256), enc_lds_bytes(R), s, a,
                     mask_k, mask_v, (int)tpw);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_all_ranks(const EncodeArgs& a, int n_heads, hipStream_t s) {
  uint64_t mk[4] = {0, 0, 0, 0}, mv[4] = {0, 0, 0, 0};
  for (int h = 0; h < n_heads; ++h) {  // vector-quantized tensors are encoded elsewhere
    const int ik = __builtin_ctz((unsigned)a.heads.h[h].rk) - 4, iv = __builtin_ctz((unsigned)a.heads.h[h].rv) - 4;
    if (!is_vq(a.heads.h[h].bk)) mk[ik] |= 1ull << h;
    if (!is_vq(a.heads.h[h].bv)) mv[iv] |= 1ull << h;
  }
  hipError_t e;
  if ((e = launch_rank<T, 16>(a, mk[0], mv[0], s)) != hipSuccess) return e;
  if ((e = launch_rank<T, 32>(a, mk[1], mv[1], s)) != hipSuccess) return e;
  if ((e = launch_rank<T, 64>(a, mk[2], mv[2], s)) != hipSuccess) return e;
  return launch_rank<T, 128>(a, mk[3], mv[3], s);
}

}  // namespace

hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  return a.dtype == 0 ? launch_all_ranks<float>(a, a.n_kv_heads, s) : launch_all_ranks<_Float16>(a, a.n_kv_heads, s);
}

}  // namespace kvtc
