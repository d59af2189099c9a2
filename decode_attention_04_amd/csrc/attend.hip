// Decode attention over the compressed cache for gfx950: query projection,
// split-K attention over packed records, and the log-sum-exp combine with
// the value back-projection.
//
// KV-COBRA project page, "Efficiency": dequantization and the inverse rotation
// run in one pass over packed b-bit codes.  pith.science NOVA-KV verdict,
// forward implications: the inverse key transform is folded into the query, so
// the score of token t is  s_t = scale * q~ . c^_t  with q~ = P_K^T q  and
// c^_t = min_t + step_t * code_t, i.e.  s_t = scale * (min_t * sum_j q~_j + step_t * q~ . code_t).
// The value side accumulates  sum_t p_t c^_V,t = (sum_t p_t min_t) 1 + sum_t (p_t step_t) code_t
// in rank-r_V space and back-projects once per query head: o = P_V o~ / l.
#include "kvtc_common.h"
#include "kvtc_launch.h"

namespace kvtc {

constexpr int kTile = 256;  // tokens per workgroup iteration (one per thread in the score phase)

// ----------------------------------------------------------------- query projection
// q~ = scale * log2(e) * P_K^T q for every (sequence, query head); S_q = sum_j q~_j.
template <typename T>
__global__ __launch_bounds__(128) void qproj_kernel(AttendArgs a) {
  __shared__ float qs[kHeadDim];
  __shared__ float red[2];
  const int bq = blockIdx.x;
  const int tid = threadIdx.x;
  const int hq = bq % a.n_q_heads;
  const HeadDesc& hd = a.heads.h[hq / a.group];
  const int r = hd.rk;
  qs[tid] = (float)((const T*)a.q)[(int64_t)bq * kHeadDim + tid];
  __syncthreads();
  float acc = 0.0f;
  if (tid < r) {
    const float* P = a.basis_k + hd.boff_k;
    for (int i = 0; i < kHeadDim; ++i) acc = fmaf(P[i * r + tid], qs[i], acc);
    acc *= a.scale_log2;
    a.qt[(int64_t)bq * kQtStride + tid] = acc;
  }
  float s = acc;
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) a.sq[bq] = red[0] + red[1];
}

// ----------------------------------------------------------------- block reductions
__device__ inline void allreduce16(float* v, int g, float* red, bool is_max) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    if (hh < g) {
      float x = v[hh];
      for (int o = 32; o > 0; o >>= 1) {
        float y = __shfl_xor(x, o);
        x = is_max ? fmaxf(x, y) : x + y;
      }
      v[hh] = x;
      if (lane == 0) red[wave * kMaxGroup + hh] = x;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    if (hh < g) {
      float x = red[hh];
      for (int w = 1; w < 4; ++w) {
        float y = red[w * kMaxGroup + hh];
        x = is_max ? fmaxf(x, y) : x + y;
      }
      v[hh] = x;
    }
  }
  __syncthreads();
}

// ----------------------------------------------------------------- score phase (thread = token)
template <int BK>
__device__ inline void score_token(const uint32_t* __restrict__ rec, int r, int g, const float* qt_lds,
                                   const float* sq, float* s) {
  float dot[kMaxGroup];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) dot[hh] = 0.0f;
  const uint32_t w0 = rec[0];
  const float mu = f16_bits_to_f32(w0 & 0xFFFFu), sg = f16_bits_to_f32(w0 >> 16);
  const int nwords = (r * BK + 31) / 32;
  uint64_t buf = 0;
  int nb = 0, j = 0;
  for (int w = 0; w < nwords; ++w) {
    buf |= (uint64_t)rec[1 + w] << nb;
    nb += 32;
    while (nb >= BK && j < r) {
      const float cf = (float)(uint32_t)(buf & ((1u << BK) - 1u));
      buf >>= BK;
      nb -= BK;
      const float* qj = qt_lds + j * kMaxGroup;
#pragma unroll
      for (int hh = 0; hh < kMaxGroup; ++hh)
        if (hh < g) dot[hh] = fmaf(qj[hh], cf, dot[hh]);
      ++j;
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh)
    if (hh < g) s[hh] = fmaf(sg, dot[hh], mu * sq[hh]);
}

// ----------------------------------------------------------------- value phase (thread = code index)
template <int BV>
__device__ inline void value_tile(const uint32_t* vrec, int wv, int jj, int tg, int ngroups, int g,
                                  const float* p_lds, float* acc) {
  const int bit = jj * BV, w = 1 + (bit >> 5), off = bit & 31;
  const bool straddle = off + BV > 32;
  for (int t = tg; t < kTile; t += ngroups) {
    const uint32_t* rw = vrec + t * wv;
    uint32_t v = rw[w] >> off;
    if (straddle) v |= rw[w + 1] << (32 - off);
    const float cf = (float)(v & ((1u << BV) - 1u));
    const float* pt = p_lds + t * kMaxGroup;
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh)
      if (hh < g) acc[hh] = fmaf(pt[hh], cf, acc[hh]);
  }
}

// ----------------------------------------------------------------- split-K attention (VALU)
// Grid (n_splits, n_kv_heads, batch), 256 threads.  The g query heads of a KV
// head share every pass over its records.  Per 256-token tile: each thread
// scores one token for all g heads, the block updates the online-softmax
// state, then threads own (code index, token group) pairs for the values.
__global__ __launch_bounds__(256) void attend_valu_kernel(AttendArgs a) {
  __shared__ float qt_lds[kMaxRank * kMaxGroup];
  __shared__ float p_lds[kTile * kMaxGroup];
  __shared__ uint32_t vrec[kTile * kMaxWords];
  __shared__ float red[4 * kMaxGroup];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const HeadDesc& hd = a.heads.h[h];
  const int g = a.group, rk = hd.rk, bk = hd.bk, rv = hd.rv, bv = hd.bv, wk = hd.wk, wv = hd.wv;
  const int64_t t_begin = (int64_t)split * a.split_tokens;
  int64_t t_end = t_begin + a.split_tokens;
  if (t_end > a.n_tokens) t_end = a.n_tokens;
  const int hq0 = h * g;
  const int64_t bq0 = (int64_t)b * a.n_q_heads + hq0;

  for (int i = tid; i < kMaxRank * kMaxGroup; i += 256) {
    const int j = i / kMaxGroup, hh = i % kMaxGroup;
    qt_lds[i] = (hh < g && j < rk) ? a.qt[(bq0 + hh) * kQtStride + j] : 0.0f;
  }
  float sq[kMaxGroup];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) sq[hh] = hh < g ? a.sq[bq0 + hh] : 0.0f;

  float m_run[kMaxGroup], l_run[kMaxGroup], c_run[kMaxGroup], acc[kMaxGroup];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.0f;
    c_run[hh] = 0.0f;
    acc[hh] = 0.0f;
  }
  const int ngroups = kTile / rv;
  const int jj = tid % rv, tg = tid / rv;
  const uint32_t* kbase = a.cache_k + hd.base_k + (int64_t)b * a.capacity * wk;
  const uint32_t* vbase = a.cache_v + hd.base_v + (int64_t)b * a.capacity * wv;
  __syncthreads();

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int64_t t = t0 + tid;
    const bool valid = t < t_end;
    float s[kMaxGroup];
    float muv = 0.0f, sgv = 0.0f;
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) s[hh] = -__builtin_inff();
    if (valid) {
      const uint32_t* rk_ = kbase + t * wk;
      switch (bk) {
        case 2: score_token<2>(rk_, rk, g, qt_lds, sq, s); break;
        case 3: score_token<3>(rk_, rk, g, qt_lds, sq, s); break;
        case 4: score_token<4>(rk_, rk, g, qt_lds, sq, s); break;
        case 5: score_token<5>(rk_, rk, g, qt_lds, sq, s); break;
        case 6: score_token<6>(rk_, rk, g, qt_lds, sq, s); break;
        case 7: score_token<7>(rk_, rk, g, qt_lds, sq, s); break;
        default: score_token<8>(rk_, rk, g, qt_lds, sq, s); break;
      }
      const uint32_t* rv_ = vbase + t * wv;
      for (int w = 0; w < wv; ++w) vrec[tid * wv + w] = rv_[w];
      muv = f16_bits_to_f32(vrec[tid * wv] & 0xFFFFu);
      sgv = f16_bits_to_f32(vrec[tid * wv] >> 16);
    }
    // online softmax update (log2 domain)
    float tmax[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) tmax[hh] = s[hh];
    allreduce16(tmax, g, red, true);
    float p[kMaxGroup], pm[kMaxGroup], alpha[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      if (hh < g) {
        const float m_new = fmaxf(m_run[hh], tmax[hh]);
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        alpha[hh] = exp2f(m_run[hh] - m_use);
        p[hh] = exp2f(s[hh] - m_use);
        pm[hh] = p[hh] * muv;
        p_lds[tid * kMaxGroup + hh] = p[hh] * sgv;
        m_run[hh] = m_new;
      }
    }
    allreduce16(p, g, red, false);
    allreduce16(pm, g, red, false);
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      if (hh < g) {
        l_run[hh] = fmaf(l_run[hh], alpha[hh], p[hh]);
        c_run[hh] = fmaf(c_run[hh], alpha[hh], pm[hh]);
        acc[hh] *= alpha[hh];
      }
    }
    // (allreduce16 ended with a barrier: p_lds and vrec are complete)
    switch (bv) {
      case 2: value_tile<2>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      case 3: value_tile<3>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      case 4: value_tile<4>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      case 5: value_tile<5>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      case 6: value_tile<6>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      case 7: value_tile<7>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
      default: value_tile<8>(vrec, wv, jj, tg, ngroups, g, p_lds, acc); break;
    }
    __syncthreads();
  }

  // reduce the value accumulators over token groups, write the split partial
  float* scratch = reinterpret_cast<float*>(vrec);
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh)
    if (hh < g) scratch[(tg * kMaxGroup + hh) * rv + jj] = acc[hh];
  __syncthreads();
  float* part0 = a.part + (bq0 * a.n_splits + split) * (int64_t)kPartStride;
  for (int o = tid; o < g * rv; o += 256) {
    const int hh = o / rv, j = o % rv;
    float sum = 0.0f;
    for (int gg = 0; gg < ngroups; ++gg) sum += scratch[(gg * kMaxGroup + hh) * rv + j];
    float cst = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxGroup; ++k)
      if (k == hh) cst = c_run[k];
    part0[(int64_t)hh * a.n_splits * kPartStride + 2 + j] = sum + cst;
  }
  if (tid < g) {
    float mm = 0.0f, ll = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxGroup; ++k)
      if (k == tid) { mm = m_run[k]; ll = l_run[k]; }
    part0[(int64_t)tid * a.n_splits * kPartStride + 0] = mm;
    part0[(int64_t)tid * a.n_splits * kPartStride + 1] = ll;
  }
}

// ----------------------------------------------------------------- combine + back-projection
// Grid: batch * n_q_heads, 128 threads (one per output dimension).
__global__ __launch_bounds__(128) void combine_kernel(AttendArgs a) {
  __shared__ float ot[kMaxRank];
  __shared__ float red[2];
  const int bq = blockIdx.x, tid = threadIdx.x;
  if (a.n_tokens <= 0) {  // attention over no tokens is defined as zero output
    a.out[(int64_t)bq * kHeadDim + tid] = 0.0f;
    return;
  }
  const int hq = bq % a.n_q_heads;
  const HeadDesc& hd = a.heads.h[hq / a.group];
  const int rv = hd.rv;
  const int ns = a.n_splits;
  const float* part = a.part + (int64_t)bq * ns * kPartStride;
  float M = -__builtin_inff();
  for (int s = tid; s < ns; s += 128) M = fmaxf(M, part[(int64_t)s * kPartStride]);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  const float m_use = M == -__builtin_inff() ? 0.0f : M;
  float L = 0.0f;
  for (int s = tid; s < ns; s += 128) {
    const float* ps = part + (int64_t)s * kPartStride;
    L += exp2f(ps[0] - m_use) * ps[1];
  }
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  if ((tid & 63) == 0) red[tid >> 6] = L;
  __syncthreads();
  L = red[0] + red[1];
  if (tid < rv) {
    float o = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float* ps = part + (int64_t)s * kPartStride;
      o = fmaf(exp2f(ps[0] - m_use), ps[2 + tid], o);
    }
    ot[tid] = o;
  }
  __syncthreads();
  float res = 0.0f;
  if (L > 0.0f) {
    const float* P = a.basis_v + hd.boff_v + (int64_t)tid * rv;
    for (int j = 0; j < rv; ++j) res = fmaf(P[j], ot[j], res);
    res /= L;
  }
  a.out[(int64_t)bq * kHeadDim + tid] = res;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  const unsigned nbq = (unsigned)(a.batch * a.n_q_heads);
  if (a.dtype == 0)
    hipLaunchKernelGGL(qproj_kernel<float>, dim3(nbq), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(qproj_kernel<_Float16>, dim3(nbq), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_tokens > 0) {
    hipLaunchKernelGGL(attend_valu_kernel, dim3(a.n_splits, a.n_kv_heads, a.batch), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(combine_kernel, dim3(nbq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvtc
