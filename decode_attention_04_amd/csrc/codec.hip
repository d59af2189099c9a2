// Encode side of the codec for gfx950: the one-token append kernel, plus the
// standalone quantize/pack and unpack kernels behind the test entry points
// (the prefill encoder is in encode_mfma.hip).
//
// KV-COBRA project page, "How KV-COBRA Works" (Inference): each key is rotated
// and truncated with the head's basis and quantized with its head's b-bit
// quantizer.  The quantizer's rounding decisions are taken with float64
// semantics (MI355X runs fp64 FMA at half the fp32 rate), from a float64
// projection summed in one fixed order.
#include "encode_core.h"
#include "kvtc_common.h"
#include "kvtc_launch.h"

namespace kvtc {

// ----------------------------------------------------------------- pack / unpack
// One wave per token: lanes hold coordinates, reduce min/max, quantize, pack.
__global__ __launch_bounds__(256) void quantize_pack_kernel(const float* __restrict__ coords, int64_t n,
                                                            int r, int b, uint32_t* __restrict__ records) {
  __shared__ uint32_t codes_lds[4][kMaxRank];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= n) return;
  const float* c = coords + t * r;
  double v0 = lane < r ? (double)c[lane] : 0.0;
  double v1 = lane + 64 < r ? (double)c[lane + 64] : 0.0;
  double mn = lane < r ? v0 : __builtin_inf(), mx = lane < r ? v0 : -__builtin_inf();
  if (lane + 64 < r) { mn = fmin(mn, v1); mx = fmax(mx, v1); }
  for (int o = 32; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o));
    mx = fmax(mx, __shfl_xor(mx, o));
  }
  QuantHeader qh = quant_header(mn, mx, b);
  if (lane < r) codes_lds[wave][lane] = quant_code(v0, qh.mu, qh.sigma, b);
  if (lane + 64 < r) codes_lds[wave][lane + 64] = quant_code(v1, qh.mu, qh.sigma, b);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const int W = record_words(r, b);
  uint32_t* rec = records + t * W;
  if (lane == 0) rec[0] = qh.word0;
  if (lane < W - 1) rec[1 + lane] = pack_word(codes_lds[wave], r, b, lane);
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ records, int64_t n, int r,
                                                     int b, uint16_t* __restrict__ min_step,
                                                     uint8_t* __restrict__ codes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * r) return;
  const int64_t t = i / r;
  const int j = (int)(i - t * r);
  const int W = record_words(r, b);
  const uint32_t* rec = records + t * W;
  codes[i] = (uint8_t)unpack_code(rec + 1, j, b);
  if (j == 0) {
    min_step[2 * t] = (uint16_t)(rec[0] & 0xFFFFu);
    min_step[2 * t + 1] = (uint16_t)(rec[0] >> 16);
  }
}

// ----------------------------------------------------------------- append
// Grid (n_kv_heads, batch), 256 threads: waves 0-1 encode the sequence's new key,
// waves 2-3 its new value, each with half of its basis loads in flight at once.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(EncodeArgs a) {
  __shared__ EncodeScratch scr[2];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tensor = threadIdx.x >> 7, t = threadIdx.x & 127;
  const HeadDesc& hd = a.heads.h[h];
  const int r = tensor ? hd.rv : hd.rk, bits = tensor ? hd.bv : hd.bk, W = tensor ? hd.wv : hd.wk;
  const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
  const T* x = (const T*)(tensor ? a.v : a.k) + ((int64_t)b * a.n_kv_heads + h) * kHeadDim;
  uint32_t* rec = (tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k) + ((int64_t)b * a.capacity + a.pos0) * W;
  encode_token_128(x, P, r, bits, rec, scr[tensor], t, [] { __syncthreads(); });
}

// ----------------------------------------------------------------- launchers
hipError_t launch_quantize_pack(const float* coords, int64_t n, int r, int b, uint32_t* records,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 3) / 4));
  hipLaunchKernelGGL(quantize_pack_kernel, grid, dim3(256), 0, s, coords, n, r, b, records);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* records, int64_t n, int r, int b, uint16_t* min_step,
                         uint8_t* codes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t total = n * r;
  dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(256), 0, s, records, n, r, b, min_step, codes);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.n_tokens == 1) {  // one token per (sequence, head): the append kernel
    const dim3 grid((unsigned)a.n_kv_heads, (unsigned)a.batch);
    if (a.dtype == 0)
      hipLaunchKernelGGL(append_kernel<float>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(append_kernel<_Float16>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return launch_encode_mfma(a, s);
}

}  // namespace kvtc
