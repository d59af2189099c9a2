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

// Encode the token x[0..128) with basis P (128 x r, float32 row-major) and b-bit
// codes into `rec` (record_words(r, b, hdr) words), using 128 threads whose index
// in the group is t (0..127, two whole waves).  hdr = 1: the record starts with
// the token's fp16 min and step; hdr = 0: header-free, the codes use the head's
// fixed min and step `sw` (fp16 min | step << 16).  The caller synchronises the
// workgroup around the call (`sync` is the workgroup barrier it uses between the
// phases; all threads of the workgroup must reach it).
template <typename T, typename Sync>
__device__ __attribute__((always_inline)) inline void encode_token_128(const T* x, const float* P, int r, int bits,
                                                                        int hdr, uint32_t sw, uint32_t* rec,
                                                                        EncodeScratch& s, int t, Sync&& sync) {
  // lane layout: four consecutive columns per lane, one row group per 32 lanes
  const int c4 = t % 32, rg = t / 32;
  const bool active = 4 * c4 < r;
  constexpr int kHalf = kGroupRows / 2;  // rows loaded per batch (keeps 64 VGPRs of the basis live)
  float4 p[kHalf];
#pragma unroll
  for (int k = 0; k < kHalf; ++k)
    if (active) p[k] = *(const float4*)(P + (int64_t)(rg * kGroupRows + k) * r + 4 * c4);
  s.xs[t] = load_f64(x + t);
  sync();
  if (active) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1) {
#pragma unroll
        for (int k = 0; k < kHalf; ++k) p[k] = *(const float4*)(P + (int64_t)(rg * kGroupRows + kHalf + k) * r + 4 * c4);
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
  QuantHeader qh;
  if (t < 64) {  // one wave: coordinates j = t, t + 64
    const int lane = t;
    double c0 = 0.0, c1 = 0.0;
    if (lane < r) c0 = ((s.gs[0][lane] + s.gs[1][lane]) + s.gs[2][lane]) + s.gs[3][lane];
    if (lane + 64 < r) c1 = ((s.gs[0][lane + 64] + s.gs[1][lane + 64]) + s.gs[2][lane + 64]) + s.gs[3][lane + 64];
    double mn = lane < r ? c0 : __builtin_inf(), mx = lane < r ? c0 : -__builtin_inf();
    if (lane + 64 < r) {
      mn = fmin(mn, c1);
      mx = fmax(mx, c1);
    }
    for (int o = 32; o > 0; o >>= 1) {
      mn = fmin(mn, __shfl_xor(mn, o));
      mx = fmax(mx, __shfl_xor(mx, o));
    }
    qh = hdr ? quant_header(mn, mx, bits) : static_header(sw);
    if (lane < r) s.codes[lane] = quant_code(c0, qh.mu, qh.sigma, bits);
    if (lane + 64 < r) s.codes[lane + 64] = quant_code(c1, qh.mu, qh.sigma, bits);
  }
  sync();
  if (t < 64) {
    const int nw = record_words(r, bits, 0);
    if (t == 0 && hdr) rec[0] = qh.word0;
    if (t < nw) rec[hdr + t] = pack_word(s.codes, r, bits, t);
  }
}

}  // namespace kvtc
