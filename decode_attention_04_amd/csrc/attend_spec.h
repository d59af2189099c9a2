// Decode attention kernels specialised per record format (gfx950).
//
// The generic kernel reads each head's (rank, bits) at run time and dispatches
// the unpacking inside the tile loop; the branches and the register moves they
// force at every merge cost about as many instructions as the tile's work.  Here
// a workgroup dispatches once, on its KV head's (r_K, b_K, r_V, b_V), to a tile
// loop compiled for that format: record sizes, copy instruction counts and the
// copy wait counts are constants, and each tile is one straight instruction
// sequence.  The built-in classes hold the formats the per-head bit allocation
// picks under one budget of bits per vector (every rank of the allocation search
// with b = min(8, floor(budget / r)) >= 2), all (K, V) pairs, with per-token
// headers or header-free; the build adds one class per frozen per-layer
// allocation (frozen_layouts.txt, generated into attend_frozen.h).  A layout
// outside every class runs the generic kernel.
#pragma once

#include "attend_core.h"

namespace kvtc {

// 64-bit budget per vector (C1 picks b = min(8, floor(budget / r)))
#define KVTC_SPEC_CLASS0(X) X(0, 16, 4, 16, 4) X(1, 16, 4, 32, 2) X(2, 32, 2, 16, 4) X(3, 32, 2, 32, 2)

// 128-bit budget per vector (C1 picks b = min(8, floor(budget / r)))
#define KVTC_SPEC_CLASS1(X) X(0, 16, 8, 16, 8) X(1, 16, 8, 32, 4) X(2, 16, 8, 64, 2) X(3, 32, 4, 16, 8) X(4, 32, 4, 32, 4) X(5, 32, 4, 64, 2) X(6, 64, 2, 16, 8) X(7, 64, 2, 32, 4) X(8, 64, 2, 64, 2)

// 256-bit budget per vector (C1 picks b = min(8, floor(budget / r)))
#define KVTC_SPEC_CLASS2(X) X(0, 16, 8, 16, 8) X(1, 16, 8, 32, 8) X(2, 16, 8, 64, 4) X(3, 16, 8, 128, 2) X(4, 32, 8, 16, 8) X(5, 32, 8, 32, 8) X(6, 32, 8, 64, 4) X(7, 32, 8, 128, 2) X(8, 64, 4, 16, 8) X(9, 64, 4, 32, 8) X(10, 64, 4, 64, 4) X(11, 64, 4, 128, 2) X(12, 128, 2, 16, 8) X(13, 128, 2, 32, 8) X(14, 128, 2, 64, 4) X(15, 128, 2, 128, 2)

// 512-bit budget per vector (C1 picks b = min(8, floor(budget / r)))
#define KVTC_SPEC_CLASS3(X) X(0, 16, 8, 16, 8) X(1, 16, 8, 32, 8) X(2, 16, 8, 64, 8) X(3, 16, 8, 128, 4) X(4, 32, 8, 16, 8) X(5, 32, 8, 32, 8) X(6, 32, 8, 64, 8) X(7, 32, 8, 128, 4) X(8, 64, 8, 16, 8) X(9, 64, 8, 32, 8) X(10, 64, 8, 64, 8) X(11, 64, 8, 128, 4) X(12, 128, 4, 16, 8) X(13, 128, 4, 32, 8) X(14, 128, 4, 64, 8) X(15, 128, 4, 128, 4)

// Header-free records (one fixed quantizer per head) of the 64- and 128-bit budget formats
#define KVTC_SPEC_CLASS4(X) KVTC_SPEC_CLASS0(X)
#define KVTC_SPEC_CLASS5(X) KVTC_SPEC_CLASS1(X)

// Vector-quantized pairs (format code kVq + index bits) of the attention-aware key
// transform and the value eigenbasis: full rank at 1, 2 and 3 bits per coordinate,
// rank 64 and 32 at 2 bits per coordinate; and vector-quantized keys (2 bits per
// coordinate) with scalar-quantized values of the same rank
#define KVTC_SPEC_CLASS6(X) X(0, 128, 20, 128, 20) X(1, 128, 18, 128, 18) X(2, 128, 22, 128, 22) \
  X(3, 64, 20, 64, 20) X(4, 32, 20, 32, 20) X(5, 128, 20, 64, 20) X(6, 128, 20, 128, 2) X(7, 64, 20, 64, 4)

constexpr int kSpecClasses = 7;  // built-in classes; the frozen ones follow them

// Header words of every record a built-in class reads: 1 (per-token header word) or 0.
__host__ __device__ constexpr int spec_header(int cls) { return cls == 4 || cls == 5 ? 0 : 1; }

// Index of (rk, bk, rv, bv) in class `cls`, or -1.
__host__ inline int spec_index(int cls, int rk, int bk, int rv, int bv) {
  int found = -1;
#define KVTC_SPEC_FIND(I, RK, BK, RV, BV) \
  if (rk == RK && bk == BK && rv == RV && bv == BV) found = I;
  switch (cls) {
    case 0: KVTC_SPEC_CLASS0(KVTC_SPEC_FIND) break;
    case 1: KVTC_SPEC_CLASS1(KVTC_SPEC_FIND) break;
    case 2: KVTC_SPEC_CLASS2(KVTC_SPEC_FIND) break;
    case 3: KVTC_SPEC_CLASS3(KVTC_SPEC_FIND) break;
    case 4: KVTC_SPEC_CLASS4(KVTC_SPEC_FIND) break;
    case 5: KVTC_SPEC_CLASS5(KVTC_SPEC_FIND) break;
    case 6: KVTC_SPEC_CLASS6(KVTC_SPEC_FIND) break;
    default: break;
  }
#undef KVTC_SPEC_FIND
  return found;
}

// Copy the records of tokens [t0, min(t0 + 64, t_end)) of both regions into tile slot `slot`.
template <int WK, int WV>
__device__ __attribute__((always_inline)) inline void issue_tile(const WaveCtx& c, int t0, int t_end, int slot) {
  uint32_t* kd = c.ktile + slot * c.kbuf;
  uint32_t* vd = c.vtile + slot * c.vbuf;
  const uint32_t r0 = tile_rec(c, t0);
  if (t0 + kTileT <= t_end) {
    tile_copy_n<64u * 4u * WK>(c.rk_, r0 * 4u * WK, kd);
    tile_copy_n<64u * 4u * WV>(c.rv_, r0 * 4u * WV, vd);
  } else {
    const uint32_t nn = (uint32_t)(t_end - t0);
    tile_copy(c.rk_, r0 * 4u * WK, nn * 4u * WK, kd);
    tile_copy(c.rv_, r0 * 4u * WV, nn * 4u * WV, vd);
  }
}

// The tile loop of one wave for records of (RK, BK) keys and (RV, BV) values, with
// (HDR = 1) or without (HDR = 0, the head's fixed min and step) per-token headers.
template <int GM, int RK, int BK, int RV, int BV, int HDR>
__device__ __attribute__((always_inline)) inline void spec_tiles(const AttendArgs& a, const WaveCtx& c,
                                                                 WaveState<GM>& st) {
  constexpr int WK = HDR + (code_count(RK, BK) * code_bits(BK) + 31) / 32;
  constexpr int WV = HDR + (code_count(RV, BV) * code_bits(BV) + 31) / 32;
  constexpr int NKS = RK >= 32 ? RK / 32 : 1, NT = RV / 16;
  static_assert(!(is_vq(BK) || is_vq(BV)) || (RK >= 32 && RV >= 32 && HDR == 1),
                "vector-quantized formats: ranks >= 32, records with their scale word");
  constexpr int KI = (16 * WK + 63) / 64, VI = (16 * WV + 63) / 64;  // copy instructions of a full tile
  static_assert(KI + VI <= 63, "vmcnt range");
  const int t_begin = c.t_begin, t_end = c.t_end, nbuf = c.nbuf;
  const int lane = threadIdx.x & 63;
  const uint32_t sk = HDR ? 0u : __builtin_amdgcn_readfirstlane(a.heads.h[c.h].sk);
  const uint32_t sv = HDR ? 0u : __builtin_amdgcn_readfirstlane(a.heads.h[c.h].sv);
  // the first nbuf - 1 tiles (one with a single buffer) start streaming behind the
  // loads of the query projection
  u32x4 aq_hi[4], aq_lo[4];
  float sq[GM], kf[GM];
  project_query<GM, BK>(a, c, RK, aq_hi, aq_lo, sq, kf, [&] {
    for (int t = 0; t < (nbuf > 1 ? nbuf - 1 : 1); ++t)
      if (t_begin + t * kTileT < t_end) issue_tile<WK, WV>(c, t_begin + t * kTileT, t_end, t);
  });
  if (threadIdx.x == 0) KVTC_STAMP(c.stamp, 1);
  init_state(st);
  if (lane < 4) ((uint32_t*)c.S)[score_floats(GM) + lane] = 0u;  // zero slot
  int slot = 0;
  lds_fence();
  for (int t0 = t_begin; t0 < t_end; t0 += kTileT) {
    const int nvalid = t_end - t0 < kTileT ? t_end - t0 : kTileT;
    const int t1 = t0 + kTileT;
    const uint32_t* kt = c.ktile + slot * c.kbuf;
    const uint32_t* vt = c.vtile + slot * c.vbuf;
    // this tile is in LDS once at most the next (full) tile's copies are outstanding
    if (nbuf == 3 && t1 + kTileT <= t_end) wait_vm<KI + VI>();
    else wait_tiles();
    const int tn = t0 + (nbuf - 1) * kTileT;  // the tile whose copy starts now
    if (nbuf >= 2 && tn < t_end) {
      int sn = slot + nbuf - 1;
      sn = sn >= nbuf ? sn - nbuf : sn;
      issue_tile<WK, WV>(c, tn, t_end, sn);
    }
    progress_priority(t0, t_begin, t_end);
    // codes of record n start at word n * W + HDR: the phases take the tile shifted to n * W + 1
    k_phase<BK, NKS, GM>(kt + HDR - 1, WK, aq_hi, aq_lo, c.S, c.cbk);
    softmax_tile<GM>(kt, vt, WK, WV, HDR, HDR, sk, sv, nvalid, c.g, c.S, sq, kf, st);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 ahi, alo;
      p_operands<GM>(c.S, kk, ahi, alo);
      v_phase<BV, NT, (GM <= 8)>(vt + HDR - 1, WV, kk, ahi, alo, st.acc2, c.cbv);
    }
    lds_fence();
    if (nbuf == 1) {
      if (t1 < t_end) issue_tile<WK, WV>(c, t1, t_end, 0);  // single buffer: refill after the tile is consumed
    } else {
      slot = slot + 1 == nbuf ? 0 : slot + 1;
    }
  }
}

#define KVTC_SPEC_CASE(I, RK, BK, RV, BV) \
  case I: spec_tiles<GM, RK, BK, RV, BV, kHdr>(a, c, st); break;

// Kernel attend_NAME_kernel<GM> and launcher launch_attend_NAME of the class whose
// formats LIST(X) enumerates, with HDR header words per record.
#define KVTC_DEFINE_ATTEND_CLASS(NAME, LIST, HDR)                                                    \
  template <int GM>                                                                                  \
  __global__ __launch_bounds__(256, 3) void attend_##NAME##_kernel(AttendArgs a) {                  \
    constexpr int kHdr = (HDR);                                                                      \
    attend_body<GM>(a, [&](const WaveCtx& c, WaveState<GM>& st) {                                    \
      switch (__builtin_amdgcn_readfirstlane(head_desc(a.heads, c.h).spec)) {                                \
        LIST(KVTC_SPEC_CASE) default : break;                                                        \
      }                                                                                              \
    });                                                                                              \
  }                                                                                                  \
  hipError_t launch_attend_##NAME(const AttendArgs& a, hipStream_t s) {                             \
    const size_t lds = attend_lds_bytes(a.kbuf_words, a.vbuf_words, a.nbuf, a.group) + 4u * a.cb_words; \
    const dim3 grid((unsigned)(a.wg_per_row * a.batch));                                          \
    if (a.group <= 4)                                                                                \
      hipLaunchKernelGGL(attend_##NAME##_kernel<4>, grid, dim3(256), lds, s, a);                    \
    else                                                                                             \
      hipLaunchKernelGGL(attend_##NAME##_kernel<8>, grid, dim3(256), lds, s, a);                    \
    return hipGetLastError();                                                                        \
  }

#define KVTC_DEFINE_SPEC_CLASS(CLS) KVTC_DEFINE_ATTEND_CLASS(spec##CLS, KVTC_SPEC_CLASS##CLS, spec_header(CLS))

}  // namespace kvtc
