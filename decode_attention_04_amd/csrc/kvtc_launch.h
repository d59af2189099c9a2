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
  const uint32_t* cb_k;  // codebooks of vector-quantized K / V records (else null)
  const uint32_t* cb_v;
  int64_t n_tokens;
  int64_t pos0;
  int64_t capacity;
  Paging pg;
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
  const uint32_t* cb_k;  // codebooks of vector-quantized K / V records (else null)
  const uint32_t* cb_v;
  float* out;
  uint32_t* cnt; // [batch][n_kv_heads] split arrival counters: zero on entry, left zero
  float* part;   // [batch][n_q_heads][n_splits][kPartStride] (head h fills its first heads.h[h].ns)
  uint32_t nonce;  // non-zero tag of this call, stored in every split partial it writes
  int64_t n_tokens;
  const int32_t* lengths;  // [batch] per-sequence context lengths (device), or null: n_tokens for all
  int64_t capacity;
  Paging pg;
  int64_t split_tokens;
  int32_t n_splits;    // the largest per-head split count: the stride of `part`
  int32_t wg_per_row;  // workgroups per sequence: the sum of the heads' split counts
  alignas(4) uint16_t wg0[kMaxKvHeads];  // first workgroup of head h within a sequence's run (read as 32-bit pairs)
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group;
  int32_t batch;
  int32_t dtype;
  float scale_log2;   // softmax_scale * log2(e)
  const void* k1;      // [batch][n_kv_heads][head_dim] key and value appended at append_pos
  const void* v1;      //   by the workgroup whose split holds it (append_pos < 0: no append)
  int64_t append_pos;
  int32_t append_dtype;  // 0 = f32, 1 = f16
  int32_t kbuf_words;  // LDS words per K / V record-tile buffer (set by launch_attend)
  int32_t vbuf_words;
  int32_t nbuf;        // tile buffers per wave: 2 (next tile streams in) or 1
  int32_t cb_words;    // LDS words for the codebooks of one KV head (K then V), 0 without any
  const double* rope;  // keys compressed before RoPE: DEVICE inverse frequencies [64] (else null)
#ifdef KVTC_STAMPS
  uint64_t* stamps;    // [grid][16] phase stamps of every workgroup, or null
#endif
};

struct DecodeArgs {
  HeadTable heads;
  const float* basis;     // the tensor's concatenated bases
  const uint32_t* cache;  // the tensor's cache
  const uint32_t* cb;     // the tensor's codebooks (vector-quantized records), else null
  float* out;             // [batch][n_kv_heads][n_tokens][head_dim]
  int64_t n_tokens;
  int64_t pos0;
  int64_t capacity;
  Paging pg;
  int32_t n_kv_heads;
  int32_t batch;
  int32_t which;          // 0 = K, 1 = V
};

// Kernel arguments travel in the kernarg segment, at most 4 KB.
static_assert(sizeof(AttendArgs) <= 4096, "AttendArgs exceeds the kernel argument limit");
static_assert(sizeof(EncodeArgs) <= 4096, "EncodeArgs exceeds the kernel argument limit");
static_assert(sizeof(DecodeArgs) <= 4096, "DecodeArgs exceeds the kernel argument limit");

hipError_t launch_quantize_pack(const float* coords, int64_t n, int r, int b, uint32_t* records,
                                hipStream_t s);
hipError_t launch_unpack(const uint32_t* records, int64_t n, int r, int b, uint16_t* min_step,
                         uint8_t* codes, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);       // records -> reconstructed vectors
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);       // one token: append kernel, else the below
hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s);  // prefill: k, v 16-byte aligned
// How a layout's decode attention runs: the specialised kernel class (-1: the
// generic kernel; built-in classes first, then the frozen ones the build generates),
// LDS tile buffers per wave and resident workgroups per CU.
struct AttendPlan {
  int spec_class = -1;
  bool gen = false;
  bool vq = false;        // some head has vector-quantized records (only the specialised classes read them)
  int cb_words = 0;       // LDS words of the largest head's codebooks
  int kbuf_words = 0, vbuf_words = 0, nbuf = 1, wg_per_cu = 1;
};
AttendPlan plan_attend(const HeadTable& heads, int n_kv_heads, int group, bool rope = false);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
// Decode attention over keys compressed before RoPE (a.rope set; group <= 8, scalar records).
hipError_t launch_attend_rope(const AttendArgs& a, hipStream_t s);
// Decode attention specialised for the record formats of one class (group <= 8).
hipError_t launch_attend_spec0(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec1(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec2(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec3(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec4(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec5(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_spec6(const AttendArgs& a, hipStream_t s);

}  // namespace kvtc
