// One v_mfma_f32_16x16x32_f16 per problem on caller-given operands: the instruction
// whose arithmetic the prefill encoder's error bound and the decode kernels' code
// operands rest on (products of fp16 values, fp16 subnormals among them, summed and
// added to an fp32 accumulator).  Measurement only: not part of the decode path or
// of the kvtc library; the tests read its results against exact sums.
//
// Operand layout of the instruction on gfx950 (wave64): lane l holds A row l % 16,
// elements k = 8 (l / 16) .. 8 (l / 16) + 7; B column l % 16, the same k; and D
// column l % 16, rows 4 (l / 16) .. 4 (l / 16) + 3.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 probe_f16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));

// Problem p = blockIdx.x: a [16][32], b [32][16], c and d [16][16], row-major.
__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint16_t* a, const uint16_t* b, const float* c,
                                                        float* d) {
  const int p = blockIdx.x, l = threadIdx.x, i = l & 15, g = l >> 4;
  const uint16_t* ap = a + (int64_t)p * 512;
  const uint16_t* bp = b + (int64_t)p * 512;
  const float* cp = c + (int64_t)p * 256;
  float* dp = d + (int64_t)p * 256;
  probe_f16x8 av, bv;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    av[k] = __builtin_bit_cast(_Float16, ap[i * 32 + 8 * g + k]);
    bv[k] = __builtin_bit_cast(_Float16, bp[(8 * g + k) * 16 + i]);
  }
  probe_f32x4 cv;
#pragma unroll
  for (int e = 0; e < 4; ++e) cv[e] = cp[(4 * g + e) * 16 + i];
  const probe_f32x4 dv = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, cv, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) dp[(4 * g + e) * 16 + i] = dv[e];
}

}  // namespace

// n problems (n >= 1), device pointers; returns the launch status (0 on success).
extern "C" int kvtc_mfma_probe(const uint16_t* a, const uint16_t* b, const float* c, float* d, int n,
                               void* stream) {
  if (n < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)n), dim3(64), 0, (hipStream_t)stream, a, b, c, d);
  return (int)hipGetLastError();
}
