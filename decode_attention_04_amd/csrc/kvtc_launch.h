// Kernel argument blocks and launchers of the kvtc library (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvtc_common.h"

namespace kvtc {

struct EncodeArgs {
  HeadTable heads;
  const void* k;
  const void* v;
  const float* basis_k;
  const float* basis_v;
  uint32_t* cache_k;
  uint32_t* cache_v;
  int64_t n_tokens;
  int64_t pos0;
  int64_t capacity;
  int32_t n_kv_heads;
  int32_t batch;
  int32_t dtype;  // 0 = f32, 1 = f16
};

struct AttendArgs {
  HeadTable heads;
  const void* q;
  const float* basis_k;
  const float* basis_v;
  const uint32_t* cache_k;
  const uint32_t* cache_v;
  float* out;
  float* qt;     // [batch][n_q_heads][kQtStride] projected, pre-scaled queries
  float* sq;     // [batch][n_q_heads] sum of the projected query
  float* part;   // [batch][n_q_heads][n_splits][kPartStride]
  int64_t n_tokens;
  int64_t capacity;
  int64_t split_tokens;
  int32_t n_splits;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group;
  int32_t batch;
  int32_t dtype;
  float scale_log2;   // softmax_scale * log2(e)
  int32_t kbuf_words;  // LDS words per K / V record-tile buffer (set by launch_attend)
  int32_t vbuf_words;
  int32_t nbuf;        // tile buffers per wave: 2 (next tile streams in) or 1
};

hipError_t launch_quantize_pack(const float* coords, int64_t n, int r, int b, uint32_t* records,
                                hipStream_t s);
hipError_t launch_unpack(const uint32_t* records, int64_t n, int r, int b, uint16_t* min_step,
                         uint8_t* codes, hipStream_t s);
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace kvtc
