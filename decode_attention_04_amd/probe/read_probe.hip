// A plain streaming read of device memory: the measured HBM read rate of the GPU
// it runs on, against which the decode kernels' rates are set (beside the 8 TB/s
// datasheet peak).  Each workgroup reads one contiguous chunk with 16-byte
// non-temporal loads, four in flight per thread, and folds them into a value that
// it stores only when it equals a constant the data never produces (so the loads
// cannot be dropped and nothing is written).  Measurement only: not part of the
// decode path or of the kvtc library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const probe_u32x4* __restrict__ p, uint64_t n_vec,
                                                         uint64_t per_wg, uint32_t* sink) {
  const uint64_t b0 = (uint64_t)blockIdx.x * per_wg;
  const uint64_t b1 = b0 + per_wg < n_vec ? b0 + per_wg : n_vec;
  uint32_t acc = 0u;
  for (uint64_t i = b0 + threadIdx.x; i < b1; i += 256 * 4) {
    probe_u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = i + 256 * u < b1 ? __builtin_nontemporal_load(p + i + 256 * u) : probe_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) at device address p with `wgs` workgroups on
// `stream`; sink: device memory of at least 4 * wgs bytes.  Returns the HIP error code.
extern "C" int kvtc_read_probe(const void* p, uint64_t bytes, int32_t wgs, uint32_t* sink, void* stream) {
  if (!p || !sink || wgs <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  const uint64_t n_vec = bytes / 16;
  const uint64_t per_wg = (n_vec + (uint64_t)wgs - 1) / (uint64_t)wgs;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream,
                     (const probe_u32x4*)p, n_vec, per_wg, sink);
  return (int)hipGetLastError();
}
