// Device building blocks of the encoder (gfx950): the float64 projection of a
// token onto its head's basis in one fixed summation order, and the encode of a
// single token by 128 threads with half of its basis loads in flight at once (append).
//
// KV-COBRA project page, "How KV-COBRA Works" (Inference): each key is rotated
// and truncated with the head's basis and quantized with its head's b-bit
// quantizer.  Summation order: the 128 rows of the basis in four groups of 32,
// each accumulated in row order with fused multiply-adds, then the group sums
// added in group order.  Every encode path uses this order, so a token's record
// does not depend on the path (prefill, append, or append fused with attention)
// that wrote it.
#pragma once

#include "kvtc_common.h"

namespace kvtc {

constexpr int kRowGroups = 4;
constexpr int kGroupRows = kHeadDim / kRowGroups;  // 32

template <typename T>
__device__ inline double load_f64(const T* p) {
  return (double)(float)(*p);
}

// LDS scratch of one encode_token_128 call (one tensor).
struct EncodeScratch {
  double xs[kHeadDim];                 // the token
  double gs[kRowGroups][kMaxRank];     // group sums of the projection
  uint32_t codes[kMaxRank];
};

// Vector quantization of one token's coordinates c[0..r) (float64, in LDS) by one
// wave: rho = fp16(sqrt(mean c^2)) (lane sums c_lane^2 + c_(lane+64)^2, then a
// butterfly over the wave), u = c / rho (0 when rho = 0), and lane j < r/2 picks for
// pair (2j, 2j + 1) the nearest of its 2^bits codewords cb[j 2^bits + e] (fp16 even |
// odd << 16) by the float64 distance (u_2j - w0)^2 + (u_2j+1 - w1)^2 (each square and
// the sum rounded once), the first one on ties.  Every encode path takes these steps
// through the helpers below, so their records agree bit for bit.

// fp16 bits of the token's RMS scale rho (wave-uniform).
__device__ inline uint32_t vq_scale_bits(const double* c, int lane, int r) {
  const double c0 = lane < r ? c[lane] : 0.0, c1 = lane + 64 < r ? c[lane + 64] : 0.0;
  double sq = __dadd_rn(__dmul_rn(c0, c0), __dmul_rn(c1, c1));
  for (int o = 32; o > 0; o >>= 1) sq = __dadd_rn(sq, __shfl_xor(sq, o));
  return f64_to_f16_rne(__builtin_sqrt(sq / (double)r));
}

// The normalised coordinates of pair `lane` (lane < r/2).
__device__ inline void vq_pair_inputs(const double* c, int lane, uint32_t rb, double& u0, double& u1) {
  const double rho = (double)f16_bits_to_f32(rb);
  u0 = rho > 0.0 ? c[2 * lane] / rho : 0.0;
  u1 = rho > 0.0 ? c[2 * lane + 1] / rho : 0.0;
}

// Float64 squared distance of (u0, u1) to codeword w, each square and the sum rounded once.
__device__ inline double vq_dist(double u0, double u1, uint32_t w) {
  const double d0 = u0 - (double)f16_bits_to_f32(w & 0xFFFFu);
  const double d1 = u1 - (double)f16_bits_to_f32(w >> 16);
  return __dadd_rn(__dmul_rn(d0, d0), __dmul_rn(d1, d1));
}

// Index of the codeword nearest (u0, u1) among the K >= 4 at w (memory), the first on
// ties; eight codewords' loads at a time.
__device__ inline int vq_nearest(double u0, double u1, const uint32_t* w, int K) {
  double best = __builtin_inf();
  int bi = 0;
  for (int e0 = 0; e0 < K; e0 += 8) {
    uint32_t we[8];
#pragma unroll
    for (int u8 = 0; u8 < 8; ++u8) we[u8] = e0 + u8 < K ? w[e0 + u8] : 0u;
#pragma unroll
    for (int u8 = 0; u8 < 8; ++u8) {
      if (e0 + u8 >= K) break;
      const double dist = vq_dist(u0, u1, we[u8]);
      if (dist < best) {
        best = dist;
        bi = e0 + u8;
      }
    }
  }
  return bi;
}

// The same search over K codewords held in registers.
template <int K>
__device__ inline int vq_nearest_regs(double u0, double u1, const uint32_t (&w)[K]) {
  double best = __builtin_inf();
  int bi = 0;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const double dist = vq_dist(u0, u1, w[e]);
    if (dist < best) {
      best = dist;
      bi = e;
    }
  }
  return bi;
}

// One token by one wave, codebook in memory: indices to codes[j]; returns the header
// word (fp16 +0 | fp16 rho << 16).
__device__ inline uint32_t vq_encode_wave(const double* c, int lane, int r, int bits, const uint32_t* cb,
                                          uint32_t* codes) {
  const uint32_t rb = vq_scale_bits(c, lane, r);
  if (2 * lane < r) {
    double u0, u1;
    vq_pair_inputs(c, lane, rb, u0, u1);
    const int K = 1 << bits;
    codes[lane] = (uint32_t)vq_nearest(u0, u1, cb + (int64_t)lane * K, K);
  }
  return rb << 16;
}

// Encode the token x[0..128) with basis P (128 x r, float32 row-major) into `rec`
// (format_words(r, B, hdr) words), using 128 threads whose index in the group is t
// (0..127, two whole waves).  B: b-bit scalar codes (2..8), or kVq + b for
// vector-quantized pairs with the tensor's codebook of this head at `cb`.  hdr = 1:
// the record starts with the token's header word (fp16 min and step, or +0 and rho);
// hdr = 0: header-free scalar codes with the head's fixed min and step `sw` (fp16
// min | step << 16).  The caller synchronises the workgroup around the call (`sync`
// is the workgroup barrier it uses between the phases; all threads of the workgroup
// must reach it).
template <typename T, typename Sync>
__device__ __attribute__((always_inline)) inline void encode_token_128(const T* x, const float* P, int r, int B,
                                                                        int hdr, uint32_t sw, const uint32_t* cb,
                                                                        uint32_t* rec, EncodeScratch& s, int t,
                                                                        Sync&& sync) {
  const int bits = code_bits(B);
  // lane layout: four consecutive columns per lane, one row group per 32 lanes
  const int c4 = t % 32, rg = t / 32;
  const bool active = 4 * c4 < r;
  // lanes past the rank re-read columns 0..3 and drop them: with no load conditional,
  // a batch's loads are all in flight before the first use (a load under a lane mask
  // is followed by its own wait)
  const int col = active ? 4 * c4 : 0;
  constexpr int kHalf = kGroupRows / 2;  // rows loaded per batch (keeps 64 VGPRs of the basis live)
  float4 p[kHalf];
#pragma unroll
  for (int k = 0; k < kHalf; ++k) p[k] = *(const float4*)(P + (int64_t)(rg * kGroupRows + k) * r + col);
  s.xs[t] = load_f64(x + t);
  sync();
  if (active) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1) {
#pragma unroll
        for (int k = 0; k < kHalf; ++k) p[k] = *(const float4*)(P + (int64_t)(rg * kGroupRows + kHalf + k) * r + col);
      }
#pragma unroll
      for (int k = 0; k < kHalf; ++k) {
        const double xv = s.xs[rg * kGroupRows + half * kHalf + k];
        a0 = fma(xv, (double)p[k].x, a0);
        a1 = fma(xv, (double)p[k].y, a1);
        a2 = fma(xv, (double)p[k].z, a2);
        a3 = fma(xv, (double)p[k].w, a3);
      }
    }
    s.gs[rg][4 * c4] = a0;
    s.gs[rg][4 * c4 + 1] = a1;
    s.gs[rg][4 * c4 + 2] = a2;
    s.gs[rg][4 * c4 + 3] = a3;
  }
  sync();
  uint32_t w0 = 0u;
  if (t < 64) {  // one wave: coordinates j = t, t + 64
    const int lane = t;
    double c0 = 0.0, c1 = 0.0;
    if (lane < r) c0 = ((s.gs[0][lane] + s.gs[1][lane]) + s.gs[2][lane]) + s.gs[3][lane];
    if (lane + 64 < r) c1 = ((s.gs[0][lane + 64] + s.gs[1][lane + 64]) + s.gs[2][lane + 64]) + s.gs[3][lane + 64];
    if (is_vq(B)) {
      double* cs = s.xs;  // the token's inputs are no longer needed: its coordinates
      if (lane < r) cs[lane] = c0;
      if (lane + 64 < r) cs[lane + 64] = c1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      w0 = vq_encode_wave(cs, lane, r, bits, cb, s.codes);
    } else {
      double mn = lane < r ? c0 : __builtin_inf(), mx = lane < r ? c0 : -__builtin_inf();
      if (lane + 64 < r) {
        mn = fmin(mn, c1);
        mx = fmax(mx, c1);
      }
      for (int o = 32; o > 0; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
      }
      const QuantHeader qh = hdr ? quant_header(mn, mx, bits) : static_header(sw);
      w0 = qh.word0;
      if (lane < r) s.codes[lane] = quant_code(c0, qh.mu, qh.sigma, bits);
      if (lane + 64 < r) s.codes[lane + 64] = quant_code(c1, qh.mu, qh.sigma, bits);
    }
  }
  sync();
  if (t < 64) {
    const int nw = format_words(r, B, 0);
    if (t == 0 && hdr) rec[0] = w0;
    if (t < nw) rec[hdr + t] = pack_word(s.codes, code_count(r, B), bits, t);
  }
}

}  // namespace kvtc
