// Prefill encoder for gfx950: the (tokens x 128) by (128 x r) basis contraction
// of every (sequence, KV head, tensor) on the matrix cores, with the quantizer's
// rounding decisions kept exact.
//
// KV-COBRA project page, "How KV-COBRA Works" (Inference): each key (and value)
// is rotated and truncated with its head's basis and quantized with its head's
// b-bit quantizer; at prefill that projection is one dense contraction per head.
//
// Arithmetic.  Each basis element (fp32) is split into two fp16 parts,
// P = Ph + Pl + e with |e| <= 2^-22 |P| + 2^-25, and fp32 inputs the same way
// (fp16 inputs are exact operands).  v_mfma_f32_16x16x32_f16 forms the products
// exactly and accumulates in fp32, rounding to nearest.  With at most 256
// rounded additions of terms whose magnitudes sum to S_j = sum_i |x_i P_ij| <=
// ||x||_2 (the columns of P are orthonormal), the computed coordinate c~_j is within
//     E = 1.3125 * 2^-16 * ||x||_2
// of the exact one (the split remainders add less than 2^-20.5 ||x||_2; fp32
// inputs take three products per term, 384 additions, and E = 1.6875 * 2^-16 *
// ||x||_2 + 2^-21, the last term for inputs split below the fp16 normal range;
// they must lie inside the fp16 range, |x| < 65504).  The
// header (fp16 min and step) and the codes are monotone functions of the
// coordinates, so a decision that takes the same value at c~ - E and c~ + E is
// the exact decision.  The others are recomputed from the float64 projection in
// the fixed summation order every encode path uses (four groups of 32 rows, then
// the group sums in order):
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

// Float index, in the staged basis, of P[k][j]: the A operand (P^T, 16 coordinates
// x 32 rows) of coordinate block j/16 and row block k/32 in lane order, split in
// two planes of four rows so that every lane reads 16 contiguous bytes.
__device__ inline int basis_slot(int k, int j) {
  const int mb = j >> 4, m = j & 15, ks = k >> 5, G = (k >> 3) & 3, i = k & 7;
  return ((((mb * 4 + ks) * 2 + (i >> 2)) * 64 + 16 * G + m) << 2) + (i & 3);
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

// Exact (float64) coordinate j of the token whose 128 inputs start at `row`,
// summed in the fixed order of the encoder (rows 32q .. 32q+31 in order, q = 0..3,
// then ((g0 + g1) + g2) + g3); P is read from the staged basis.
template <typename T>
__device__ inline double exact_coord(const T* row, const float* pb, int j) {
  double g[kRowGroups];
#pragma unroll 1
  for (int q = 0; q < kRowGroups; ++q) {
    double acc = 0.0;
#pragma unroll
    for (int c8 = 0; c8 < 4; ++c8) {
      float xv[8];
      load8(row + 32 * q + 8 * c8, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fma((double)xv[i], (double)pb[basis_slot(32 * q + 8 * c8 + i, j)], acc);
    }
    g[q] = acc;
  }
  return ((g[0] + g[1]) + g[2]) + g[3];
}

// Dynamic LDS: the basis (R x 128 floats, operand order), then per wave the codes
// of one 16-token block (16 x R bytes) and its 16 header words.
__host__ __device__ constexpr int enc_wave_bytes(int R) { return 16 * R + 64; }
__host__ __device__ constexpr int enc_lds_bytes(int R) { return R * kHeadDim * 4 + kEncWaves * enc_wave_bytes(R); }

// Grid: x = groups of `tiles_per_wg` token tiles, y = the (head, tensor) units of
// rank R (keys of the heads in mask_k, then values of the heads in mask_v), z =
// sequence.  Each wave projects 16*NT tokens per tile: A = P^T from LDS (split
// into fp16 hi/lo on the fly), B = the tokens' inputs straight from HBM, one
// 16 x 16 coordinate-by-token accumulator per (coordinate block, token block).
template <typename T, int R, int NT>
__global__ __launch_bounds__(256, 2) void encode_mfma_kernel(EncodeArgs a, uint64_t mask_k, uint64_t mask_v,
                                                             int tiles_per_wg) {
  constexpr int MB = R / 16;
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int kWaveTok = 16 * NT;
  constexpr int kTileTok = kEncWaves * kWaveTok;
  extern __shared__ float enc_lds[];
  float* pb = enc_lds;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* codes = (uint8_t*)(pb + R * kHeadDim) + wave * enc_wave_bytes(R);
  uint32_t* hdrw = (uint32_t*)(codes + 16 * R);

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
  const int W = tensor ? hd.wv : hd.wk;
  const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
  const T* xu = (const T*)(tensor ? a.v : a.k) + ((int64_t)b * a.n_kv_heads + h) * a.n_tokens * kHeadDim;
  uint32_t* cu = (tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k) + ((int64_t)b * a.capacity + a.pos0) * W;

  // stage the basis in operand order (four rows of one column per thread and step)
  for (int q = tid; q < R * 32; q += 256) {
    const int ln = q & 63, hf = (q >> 6) & 1, ks = (q >> 7) & 3, mb = q >> 9;
    const int k0 = 32 * ks + 8 * (ln >> 4) + 4 * hf, j = 16 * mb + (ln & 15);
    float4 v;
    v.x = P[(k0 + 0) * R + j];
    v.y = P[(k0 + 1) * R + j];
    v.z = P[(k0 + 2) * R + j];
    v.w = P[(k0 + 3) * R + j];
    *(float4*)(pb + 4 * q) = v;
  }
  __syncthreads();

  const float top = (float)((1 << bits) - 1);
  const int64_t n_tiles = (a.n_tokens + kTileTok - 1) / kTileTok;
#pragma unroll 1
  for (int it = 0; it < tiles_per_wg; ++it) {
    const int64_t tile = (int64_t)blockIdx.x * tiles_per_wg + it;
    if (tile >= n_tiles) break;
    const int64_t wtok0 = tile * kTileTok + wave * kWaveTok;

    // ---- B operands: lane (n, G) holds dims 32ks + 8G .. +7 of token 16nt + n
    enc_u32x4 bh[4][NT], bl[4][NT];
    float ss[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t tok = wtok0 + 16 * nt + n;
      ss[nt] = 0.f;
      const T* row = xu + tok * kHeadDim + 8 * G;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (!kF32) {
          enc_u32x4 v = {0u, 0u, 0u, 0u};
          if (tok < a.n_tokens) v = *(const enc_u32x4*)(row + 32 * ks);
          bh[ks][nt] = v;
        } else {
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
    }
    if constexpr (!kF32) {
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
        const float* pa = pb + ((((mb * 4 + ks) * 2) * 64 + lane) << 2);
        const float4 p0 = *(const float4*)pa, p1 = *(const float4*)(pa + 256);
        const float pf[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        enc_half8 ah, al;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ah[i] = (_Float16)pf[i];
          al[i] = (_Float16)(pf[i] - (float)ah[i]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mb][nt] = mma(ah, bh[ks][nt], acc[mb][nt]);
          acc[mb][nt] = mma(al, bh[ks][nt], acc[mb][nt]);
          if constexpr (kF32) acc[mb][nt] = mma(ah, bl[ks][nt], acc[mb][nt]);
        }
      }
    }

    // ---- per 16-token block: header, codes, exact recomputation near boundaries, pack
#pragma unroll 1
    for (int nt = 0; nt < NT; ++nt) {
      float c[MB * 4];
      float s2 = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t == nt) {
          s2 = ss[t];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) c[mb * 4 + i] = acc[mb][t][i];
        }
      const int64_t tok = wtok0 + 16 * nt + n;
      const bool valid = tok < a.n_tokens;
      const T* row = xu + tok * kHeadDim;
      s2 += __shfl_xor(s2, 16);
      s2 += __shfl_xor(s2, 32);
      float mn = c[0], mx = c[0];
#pragma unroll
      for (int s = 1; s < MB * 4; ++s) {
        mn = fminf(mn, c[s]);
        mx = fmaxf(mx, c[s]);
      }
      mn = fminf(mn, __shfl_xor(mn, 16));
      mn = fminf(mn, __shfl_xor(mn, 32));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // error bound of the coordinates: 256 (fp16 inputs) or 384 (fp32 inputs, three
      // products per term) rounded additions, plus the split remainders; an fp32
      // input below the fp16 normal range keeps an absolute split error of up to
      // 2^-25 per element, at most 2^-25 * ||P_j||_1 <= 2^-21.5 per coordinate
      const float E = kF32 ? 0x1.bp-16f * __builtin_sqrtf(s2) + 0x1p-21f : 0x1.5p-16f * __builtin_sqrtf(s2);

      // header from the approximate extremes, if no value within E changes it
      uint32_t w0;
      bool hok;
      {
        const double ed = (double)E, kq = (double)((1 << bits) - 1);
        const uint32_t m_lo = f64_to_f16_rne((double)mn - ed), m_hi = f64_to_f16_rne((double)mn + ed);
        const double mu = f16_bits_to_f64(m_lo);
        double r_lo = (double)mx - ed - mu, r_hi = (double)mx + ed - mu;
        if (!(r_lo > 0.0)) r_lo = 0.0;
        if (!(r_hi > 0.0)) r_hi = 0.0;
        const uint32_t s_lo = f64_to_f16_rne(r_lo / kq), s_hi = f64_to_f16_rne(r_hi / kq);
        hok = m_lo == m_hi && s_lo == s_hi;
        w0 = m_lo | (s_lo << 16);
      }
      const bool hbad = valid && !hok;
      if (__ballot(hbad)) {
        uint32_t cand = 0u;
        if (hbad) {
#pragma unroll
          for (int s = 0; s < MB * 4; ++s)
            if (c[s] <= mn + 2.f * E || c[s] >= mx - 2.f * E) cand |= 1u << s;
        }
        double emin = __builtin_inf(), emax = -__builtin_inf();
        while (__ballot(cand != 0u)) {
          if (cand) {
            const int s = __builtin_ctz(cand);
            cand &= cand - 1u;
            const double v = exact_coord(row, pb, 16 * (s >> 2) + 4 * G + (s & 3));
            emin = fmin(emin, v);
            emax = fmax(emax, v);
          }
        }
        emin = fmin(emin, __shfl_xor(emin, 16));
        emin = fmin(emin, __shfl_xor(emin, 32));
        emax = fmax(emax, __shfl_xor(emax, 16));
        emax = fmax(emax, __shfl_xor(emax, 32));
        if (hbad) w0 = quant_header(emin, emax, bits).word0;
      }
      if (G == 0) hdrw[n] = w0;

      // codes from the approximate coordinates, if no value within E changes them
      const float muf = f16_bits_to_f32(w0 & 0xFFFFu), sgf = f16_bits_to_f32(w0 >> 16);
      const bool sig_pos = sgf > 0.f;
      const float inv = sig_pos ? 1.0f / sgf : 0.f;
      const float tol = E * inv * 1.0001f + 0x1p-13f;
      uint32_t flags = 0u;
#pragma unroll
      for (int s = 0; s < MB * 4; ++s) {
        const float u = (c[s] - muf) * inv;
        const float lo = fminf(fmaxf(__builtin_floorf(u - tol + 0.5f), 0.f), top);
        const float hi = fminf(fmaxf(__builtin_floorf(u + tol + 0.5f), 0.f), top);
        codes[n * R + 16 * (s >> 2) + 4 * G + (s & 3)] = (uint8_t)lo;
        if (valid && sig_pos && lo != hi) flags |= 1u << s;
      }
      if (__ballot(flags != 0u)) {
        const double mu = (double)muf, sg = (double)sgf;
        while (__ballot(flags != 0u)) {
          if (flags) {
            const int s = __builtin_ctz(flags);
            flags &= flags - 1u;
            const int j = 16 * (s >> 2) + 4 * G + (s & 3);
            codes[n * R + j] = (uint8_t)quant_code(exact_coord(row, pb, j), mu, sg, bits);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // pack and store the block's records (consecutive tokens are contiguous)
      const int64_t btok0 = wtok0 + 16 * nt;
      for (int f = lane; f < 16 * W; f += 64) {
        const int tn = f / W, w = f - tn * W;
        if (btok0 + tn < a.n_tokens) cu[btok0 * W + f] = w == 0 ? hdrw[tn] : pack_word(codes + tn * R, R, bits, w - 1);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <typename T, int R, int NT>
hipError_t launch_rank(const EncodeArgs& a, uint64_t mask_k, uint64_t mask_v, hipStream_t s) {
  const int units = __builtin_popcountll(mask_k) + __builtin_popcountll(mask_v);
  if (units == 0) return hipSuccess;
  constexpr int kTileTok = kEncWaves * 16 * NT;
  const int64_t n_tiles = (a.n_tokens + kTileTok - 1) / kTileTok;
  // about 2048 workgroups or more in flight, each staging the basis once for its tiles
  const int64_t per_tile_row = (int64_t)units * a.batch;
  int64_t tpw = (n_tiles * per_tile_row) / 2048;
  tpw = tpw < 1 ? 1 : (tpw > 8 ? 8 : tpw);
  const dim3 grid((unsigned)((n_tiles + tpw - 1) / tpw), (unsigned)units, (unsigned)a.batch);
  hipLaunchKernelGGL((encode_mfma_kernel<T, R, NT>), grid, dim3(256), enc_lds_bytes(R), s, a, mask_k, mask_v,
                     (int)tpw);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_all_ranks(const EncodeArgs& a, int n_heads, hipStream_t s) {
  constexpr bool kF32 = sizeof(T) == 4;
  uint64_t mk[4] = {0, 0, 0, 0}, mv[4] = {0, 0, 0, 0};
  for (int h = 0; h < n_heads; ++h) {
    const int ik = __builtin_ctz((unsigned)a.heads.h[h].rk) - 4, iv = __builtin_ctz((unsigned)a.heads.h[h].rv) - 4;
    mk[ik] |= 1ull << h;
    mv[iv] |= 1ull << h;
  }
  hipError_t e;
  if ((e = launch_rank<T, 16, kF32 ? 2 : 4>(a, mk[0], mv[0], s)) != hipSuccess) return e;
  if ((e = launch_rank<T, 32, kF32 ? 2 : 4>(a, mk[1], mv[1], s)) != hipSuccess) return e;
  if ((e = launch_rank<T, 64, kF32 ? 2 : 4>(a, mk[2], mv[2], s)) != hipSuccess) return e;
  return launch_rank<T, 128, 2>(a, mk[3], mv[3], s);
}

}  // namespace

hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  return a.dtype == 0 ? launch_all_ranks<float>(a, a.n_kv_heads, s) : launch_all_ranks<_Float16>(a, a.n_kv_heads, s);
}

}  // namespace kvtc
