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
// The head's codebook of one tensor (vector-quantized records), else null.
__device__ inline const uint32_t* head_codebook(const uint32_t* cb, int B, uint32_t off) {
  return is_vq(B) ? cb + off : nullptr;
}

// Grid (n_kv_heads, batch), 256 threads: waves 0-1 encode the sequence's new key,
// waves 2-3 its new value, each with half of its basis loads in flight at once.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(EncodeArgs a) {
  __shared__ EncodeScratch scr[2];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tensor = threadIdx.x >> 7, t = threadIdx.x & 127;
  const HeadDesc& hd = a.heads.h[h];
  const int r = tensor ? hd.rv : hd.rk, B = tensor ? hd.bv : hd.bk, W = tensor ? hd.wv : hd.wk;
  const int hdr = tensor ? hd.hv : hd.hk;
  const uint32_t sw = tensor ? hd.sv : hd.sk;
  const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
  const uint32_t* cb = head_codebook(tensor ? a.cb_v : a.cb_k, B, sw);
  const T* x = (const T*)(tensor ? a.v : a.k) + ((int64_t)b * a.n_kv_heads + h) * kHeadDim;
  const int64_t ri = record_index(a.pg, a.capacity, b, a.pos0);
  if (ri < 0) return;  // the whole block: both tensors share the block table
  uint32_t* rec = (tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k) + ri * W;
  encode_token_128(x, P, r, B, hdr, sw, cb, rec, scr[tensor], t, [] { __syncthreads(); });
}

// Prefill of vector-quantized tensors.  Grid (token tiles of kVqTile, 2 n_kv_heads,
// batch), y = 2h + tensor, 256 threads; blocks of scalar-quantized tensors (which the
// matrix-core encoder writes) exit.  The block stages the head's basis in LDS once,
// then takes its tokens eight at a time: every thread forms one coordinate of four of
// them in float64 in the encoders' fixed order (rows 32q .. 32q+31 in order, then
// ((g0 + g1) + g2) + g3), and one wave per token runs the append's vector quantizer
// on them (the same scale, inputs and search, with each lane's codewords in
// registers), so the records are the append's bit for bit.
constexpr int kVqTile = 64;
constexpr int kVqChunk = 8;

inline size_t vq_prefill_lds_bytes(int rmax) {
  return (size_t)kVqChunk * kHeadDim * (sizeof(double) + sizeof(float)) + kVqChunk * 64 * sizeof(uint32_t) +
         (size_t)kHeadDim * rmax * sizeof(float);
}

// The tokens of one block.  KC > 0: the pair's 2^bits = KC codewords are read once
// into registers (lane j holds those of pair j) and every search runs from them;
// KC = 0: from memory.  The inputs of the next chunk load while the current one is
// projected and searched.
template <typename T, int KC>
__device__ __attribute__((always_inline)) inline void vq_prefill_tokens(const EncodeArgs& a, int h, int tensor, int b,
                                                                        const HeadDesc& hd) {
  extern __shared__ double vq_lds[];
  const int B = tensor ? hd.bv : hd.bk;
  const int r = tensor ? hd.rv : hd.rk, W = tensor ? hd.wv : hd.wk, bits = code_bits(B);
  const float* P = tensor ? a.basis_v + hd.boff_v : a.basis_k + hd.boff_k;
  const uint32_t* cb = (tensor ? a.cb_v : a.cb_k) + (tensor ? hd.sv : hd.sk);
  const T* xu = (const T*)(tensor ? a.v : a.k) + ((int64_t)b * a.n_kv_heads + h) * a.n_tokens * kHeadDim;
  uint32_t* region = tensor ? a.cache_v + hd.base_v : a.cache_k + hd.base_k;
  double* cs = vq_lds;                                      // [kVqChunk][128] the coordinates
  float* xs = (float*)(cs + kVqChunk * kHeadDim);           // [kVqChunk][128] the inputs (exact in fp32)
  uint32_t* codes = (uint32_t*)(xs + kVqChunk * kHeadDim);  // [kVqChunk][64] pair indices
  float* Ps = (float*)(codes + kVqChunk * 64);              // [128][r] the basis
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = 1 << bits;
  uint32_t wreg[KC > 0 ? KC : 1];
  if constexpr (KC > 0) {
    const uint32_t* w = cb + (int64_t)(2 * lane < r ? lane : 0) * KC;  // lanes past the pairs re-read pair 0
#pragma unroll
    for (int e = 0; e < KC; ++e) wreg[e] = w[e];
  }
  for (int i = tid; i < kHeadDim * r; i += 256) Ps[i] = P[i];
  const int64_t t_begin = (int64_t)blockIdx.x * kVqTile;
  const int64_t t_end = t_begin + kVqTile < a.n_tokens ? t_begin + kVqTile : a.n_tokens;
  // inputs of one chunk: element tid + 256 m of [kVqChunk][128], zero past the tokens
  constexpr int kPer = kVqChunk * kHeadDim / 256;
  float xv[kPer];
  auto fetch = [&](int64_t t0) {
    const int nt = t_end - t0 < kVqChunk ? (int)(t_end - t0) : kVqChunk;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = tid + 256 * m, k = i / kHeadDim;
      xv[m] = k < nt ? (float)load_f64(xu + (t0 + k) * kHeadDim + (i - k * kHeadDim)) : 0.0f;
    }
  };
  fetch(t_begin);
  // this thread's coordinate j of tokens 4 k0 .. 4 k0 + 3 of a chunk: one basis load serves four
  const int j = tid & 127, k0 = tid >> 7;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kVqChunk) {
    const int nt = t_end - t0 < kVqChunk ? (int)(t_end - t0) : kVqChunk;
#pragma unroll
    for (int m = 0; m < kPer; ++m) xs[tid + 256 * m] = xv[m];
    __syncthreads();  // inputs (and, on the first chunk, the basis) in LDS
    if (t0 + kVqChunk < t_end) fetch(t0 + kVqChunk);
    if (j < r) {
      const float* x = xs + 4 * k0 * kHeadDim;
      double g[4][kRowGroups];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int q = 0; q < kRowGroups; ++q) g[kk][q] = 0.0;
#pragma unroll 4
      for (int i = 0; i < kGroupRows; ++i) {
#pragma unroll
        for (int q = 0; q < kRowGroups; ++q) {
          const double p = (double)Ps[(q * kGroupRows + i) * r + j];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) g[kk][q] = fma((double)x[kk * kHeadDim + q * kGroupRows + i], p, g[kk][q]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) cs[(4 * k0 + kk) * kHeadDim + j] = ((g[kk][0] + g[kk][1]) + g[kk][2]) + g[kk][3];
    }
    __syncthreads();  // coordinates complete
    for (int k = wave; k < nt; k += 4) {  // wave-uniform: one token per wave at a time
      uint32_t* cw = codes + k * 64;
      const double* c = cs + k * kHeadDim;
      const uint32_t rb = vq_scale_bits(c, lane, r);
      if (2 * lane < r) {
        double u0, u1;
        vq_pair_inputs(c, lane, rb, u0, u1);
        if constexpr (KC > 0) cw[lane] = (uint32_t)vq_nearest_regs<KC>(u0, u1, wreg);
        else cw[lane] = (uint32_t)vq_nearest(u0, u1, cb + (int64_t)lane * K, K);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int64_t ri = record_index(a.pg, a.capacity, b, a.pos0 + t0 + k);
      if (ri >= 0) {
        uint32_t* rec = region + ri * W;
        if (lane == 0) rec[0] = rb << 16;
        if (lane < W - 1) rec[1 + lane] = pack_word(cw, r / 2, bits, lane);
      }
    }
    __syncthreads();  // before the next chunk overwrites the inputs, coordinates and codes
  }
}

template <typename T>
__global__ __launch_bounds__(256) void vq_prefill_kernel(EncodeArgs a) {
  const int h = blockIdx.y >> 1, tensor = blockIdx.y & 1, b = blockIdx.z;
  const HeadDesc hd = head_desc(a.heads, h);
  const int B = tensor ? hd.bv : hd.bk;
  if (!is_vq(B)) return;  // uniform: the whole block
  // codewords per pair held in registers for up to 16 (the compiler keeps each one's
  // float64 halves live across the token loop: 64 codewords would take 256 registers)
  switch (code_bits(B)) {
    case 2: vq_prefill_tokens<T, 4>(a, h, tensor, b, hd); break;
    case 4: vq_prefill_tokens<T, 16>(a, h, tensor, b, hd); break;
    default: vq_prefill_tokens<T, 0>(a, h, tensor, b, hd); break;
  }
}

// ----------------------------------------------------------------- reconstruction
// Grid (token blocks of 16, n_kv_heads, batch), 256 threads.  The block's
// dequantized coordinates min + step * code go to LDS (one thread per (token,
// coordinate)), then each thread forms outputs x^_i = sum_j P_ij c^_j of its
// (token, i) pairs in float32, over j in order.
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  __shared__ float ch[16][kMaxRank];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const HeadDesc& hd = a.heads.h[h];
  const int r = a.which ? hd.rv : hd.rk, B = a.which ? hd.bv : hd.bk, bits = code_bits(B);
  const int W = a.which ? hd.wv : hd.wk, hdr = a.which ? hd.hv : hd.hk;
  const uint32_t sw = a.which ? hd.sv : hd.sk;
  const float* P = a.basis + (a.which ? hd.boff_v : hd.qoff_k);  // keys: reconstructed through Q_K
  const uint32_t* reg = a.cache + (a.which ? hd.base_v : hd.base_k);
  const int nt = (int)((a.n_tokens - t0) < 16 ? (a.n_tokens - t0) : 16);
  for (int e = threadIdx.x; e < 16 * r; e += 256) {
    const int tt = e / r, j = e - tt * r;
    float v = 0.0f;
    const int64_t ri = tt < nt ? record_index(a.pg, a.capacity, b, a.pos0 + t0 + tt) : -1;
    if (ri >= 0) {  // a page outside the pool reconstructs as zeros
      const uint32_t* rec = reg + ri * W;
      const uint32_t w0 = hdr ? rec[0] : sw;
      const float mu = f16_bits_to_f32(w0 & 0xFFFFu), sg = f16_bits_to_f32(w0 >> 16);
      if (is_vq(B)) {  // rho * the pair's codeword element
        const uint32_t we = a.cb[sw + ((uint32_t)(j >> 1) << bits) + unpack_code(rec + 1, j >> 1, bits)];
        v = sg * f16_bits_to_f32((j & 1) ? we >> 16 : we & 0xFFFFu);
      } else {
        v = fmaf(sg, (float)unpack_code(rec + hdr, j, bits), mu);  // one rounding to float32
      }
    }
    ch[tt][j] = v;
  }
  __syncthreads();
  float* o = a.out + (((int64_t)b * a.n_kv_heads + h) * a.n_tokens + t0) * kHeadDim;
  for (int e = threadIdx.x; e < nt * kHeadDim; e += 256) {
    const int tt = e / kHeadDim, i = e - tt * kHeadDim;
    const float* pr = P + (int64_t)i * r;
    float acc = 0.0f;
    for (int j = 0; j < r; ++j) acc = fmaf(pr[j], ch[tt][j], acc);
    o[e] = acc;
  }
}

// ----------------------------------------------------------------- launchers
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_tokens + 15) / 16), (unsigned)a.n_kv_heads, (unsigned)a.batch);
  hipLaunchKernelGGL(decode_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

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
  bool vq = false;
  for (int h = 0; h < a.n_kv_heads; ++h) vq |= is_vq(a.heads.h[h].bk) || is_vq(a.heads.h[h].bv);
  if (vq) {  // vector-quantized tensors: float64 coordinates and the append's quantizer
    int rmax = 0;
    for (int h = 0; h < a.n_kv_heads; ++h) {
      if (is_vq(a.heads.h[h].bk) && a.heads.h[h].rk > rmax) rmax = a.heads.h[h].rk;
      if (is_vq(a.heads.h[h].bv) && a.heads.h[h].rv > rmax) rmax = a.heads.h[h].rv;
    }
    const dim3 grid((unsigned)((a.n_tokens + kVqTile - 1) / kVqTile), (unsigned)(2 * a.n_kv_heads), (unsigned)a.batch);
    const size_t lds = vq_prefill_lds_bytes(rmax);
    if (a.dtype == 0)
      hipLaunchKernelGGL(vq_prefill_kernel<float>, grid, dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL(vq_prefill_kernel<_Float16>, grid, dim3(256), lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_encode_mfma(a, s);  // the scalar-quantized tensors
}

}  // namespace kvtc
