// Split-K decode attention over packed records on CDNA4 matrix cores (gfx950).
//
// The decode step contracts every token's codes with the g query heads of its
// KV head twice:  scores s[h, t] = q~_h . code_t  (r_K per token)  and the value
// sum  o~[h, j] = sum_t (p[h, t] step_t) code[t, j]  (r_V per token).  With g
// heads sharing one pass over the records (GQA) these are dense g x r x T
// contractions; on MI355X the fp32 VALU cannot keep up with HBM for b <= 4
// (4..6 VALU ops per code against ~4.9 lane-ops per HBM byte), so both run on
// v_mfma_f32_16x16x32_f16 and the VALU only unpacks codes and runs the softmax.
//
// Code -> fp16 operand without conversion: a b-bit code sitting at bit o <= 10-b
// of a 16-bit half is the fp16 subnormal  code * 2^(o-24); masking a 32-bit word
// with the field of the same offset in both halves yields two operands in one
// VALU op.  The matrix cores take subnormal fp16 inputs without flushing them, and the 2^(o-24)
// factor is folded into the other operand (keys) or the partial (values).
//
// Precision: q~ and p*step are split into fp16 hi + lo parts, so products carry
// ~22 significant bits and accumulate in fp32.  For small GQA groups the two parts
// share one MFMA (hi in the first rows of the operand, lo in the next ones: values
// for g <= 8, scores for g <= 4); otherwise each part takes its own MFMA.
//
// Pages: KV-COBRA project page, "Efficiency" (dequantization and inverse rotation
// in one pass over packed codes); pith.science NOVA-KV verdict, forward
// implications (the inverse key transform folded into the query).
#include "attend_core.h"
#include "attend_frozen.h"
#include "attend_spec.h"

namespace kvtc {

// ktc / vtc: the tile shifted so that the codes of record n start at word n * w + 1
// (one word earlier than the tile for header-free records)
#define KVTC_K_CASE(B)                                                              \
  case B:                                                                           \
    if (nks == 1) k_phase<B, 1, GM>(ktc, wk, aq_hi, aq_lo, S);                      \
    else if (nks == 2) k_phase<B, 2, GM>(ktc, wk, aq_hi, aq_lo, S);                 \
    else k_phase<B, 4, GM>(ktc, wk, aq_hi, aq_lo, S);                               \
    break;
#define KVTC_V_CASE(B)                                                              \
  case B:                                                                           \
    if (NT == 1) v_phase<B, 1, (GM <= 8)>(vtc, wv, kk, ahi, alo, acc2);                        \
    else if (NT == 2) v_phase<B, 2, (GM <= 8)>(vtc, wv, kk, ahi, alo, acc2);                   \
    else if (NT == 4) v_phase<B, 4, (GM <= 8)>(vtc, wv, kk, ahi, alo, acc2);                   \
    else v_phase<B, 8, (GM <= 8)>(vtc, wv, kk, ahi, alo, acc2);                                \
    break;

// ----------------------------------------------------------------- generic tile loop
// Any layout: the head's widths are read at run time and every tile dispatches
// its unpacking (GEN adds the general widths 3, 5, 6, 7).
template <int GM, bool GEN>
__device__ __attribute__((always_inline)) inline void generic_tiles(const AttendArgs& a, const WaveCtx& c,
                                                                    WaveState<GM>& st) {
  const HeadDesc hd = head_desc(a.heads, c.h);
  const int rk = __builtin_amdgcn_readfirstlane(hd.rk), rv = __builtin_amdgcn_readfirstlane(hd.rv);
  const int bk = __builtin_amdgcn_readfirstlane(hd.bk), bv = __builtin_amdgcn_readfirstlane(hd.bv);
  const int wk = hd.wk, wv = hd.wv;
  const int hk = __builtin_amdgcn_readfirstlane(hd.hk), hv = __builtin_amdgcn_readfirstlane(hd.hv);
  const uint32_t skw = __builtin_amdgcn_readfirstlane(hd.sk), svw = __builtin_amdgcn_readfirstlane(hd.sv);
  const int nks = rk >= 32 ? rk / 32 : 1;
  const int NT = rv / 16;
  const int t_begin = c.t_begin, t_end = c.t_end, nbuf = c.nbuf;
  const int lane = threadIdx.x & 63;
  u32x4 aq_hi[4], aq_lo[4];
  float sq[GM], kf[GM];
  const uint32_t kl = lds_addr(c.ktile), vl = lds_addr(c.vtile);
  project_query<GM, 0>(a, c, rk, aq_hi, aq_lo, sq, kf, [&] {  // the first tiles, behind the projection loads
    for (int t = 0; t < (nbuf > 1 ? nbuf - 1 : 1); ++t) {
      const int t0 = t_begin + t * kTileT;
      if (t0 < t_end) {
        const int nn = (t_end - t0) < kTileT ? (t_end - t0) : kTileT;
        const uint32_t r0 = tile_rec(c, t0);
        tile_copy(c.rk_, r0 * 4u * wk, (uint32_t)nn * 4u * wk, kl + 4u * (uint32_t)(t * c.kbuf));
        tile_copy(c.rv_, r0 * 4u * wv, (uint32_t)nn * 4u * wv, vl + 4u * (uint32_t)(t * c.vbuf));
      }
    }
  });
  if (threadIdx.x == 0) KVTC_STAMP(c.stamp, 1);
  init_state(st);
  float* S = c.S;
  f32x4 (&acc2)[8] = st.acc2;
  if (lane < 4) ((uint32_t*)S)[score_floats(GM) + lane] = 0u;  // zero slot
  int slot = 0;
  lds_fence();
  for (int t0 = t_begin; t0 < t_end; t0 += kTileT) {
    const int nvalid = t_end - t0 < kTileT ? t_end - t0 : kTileT;
    const int t1 = t0 + kTileT;
    const uint32_t* kt = c.ktile + slot * c.kbuf;
    const uint32_t* vt = c.vtile + slot * c.vbuf;
    const uint32_t* ktc = kt + hk - 1;
    const uint32_t* vtc = vt + hv - 1;
    wait_tiles();  // this tile is in LDS (the next one is issued below)
    const int tn = t0 + (nbuf - 1) * kTileT;
    if (nbuf >= 2 && tn < t_end) {
      const int nn = (t_end - tn) < kTileT ? (t_end - tn) : kTileT;
      int sn = slot + nbuf - 1;
      sn = sn >= nbuf ? sn - nbuf : sn;
      const uint32_t rn = tile_rec(c, tn);
      tile_copy(c.rk_, rn * 4u * wk, (uint32_t)nn * 4u * wk, c.ktile + sn * c.kbuf);
      tile_copy(c.rv_, rn * 4u * wv, (uint32_t)nn * 4u * wv, c.vtile + sn * c.vbuf);
    }
    progress_priority(t0, t_begin, t_end);
    if constexpr (GEN) {
      switch (bk) {
        KVTC_K_CASE(2) KVTC_K_CASE(3) KVTC_K_CASE(4) KVTC_K_CASE(5) KVTC_K_CASE(6) KVTC_K_CASE(7) KVTC_K_CASE(8)
      }
    } else {
      switch (bk) { KVTC_K_CASE(2) KVTC_K_CASE(4) KVTC_K_CASE(8) }
    }
    softmax_tile<GM>(kt, vt, wk, wv, hk, hv, skw, svw, nvalid, c.g, S, sq, kf, st);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 ahi, alo;
      p_operands<GM>(S, kk, ahi, alo);
      if constexpr (GEN) {
        switch (bv) {
          KVTC_V_CASE(2) KVTC_V_CASE(3) KVTC_V_CASE(4) KVTC_V_CASE(5) KVTC_V_CASE(6) KVTC_V_CASE(7) KVTC_V_CASE(8)
        }
      } else {
        switch (bv) { KVTC_V_CASE(2) KVTC_V_CASE(4) KVTC_V_CASE(8) }
      }
    }
    lds_fence();
    if (nbuf == 1) {
      if (t1 < t_end) {  // single buffer: refill after the tile is consumed
        const int n1 = (t_end - t1) < kTileT ? (t_end - t1) : kTileT;
        const uint32_t r1 = tile_rec(c, t1);
        tile_copy(c.rk_, r1 * 4u * wk, (uint32_t)n1 * 4u * wk, c.ktile);
        tile_copy(c.rv_, r1 * 4u * wv, (uint32_t)n1 * 4u * wv, c.vtile);
      }
    } else {
      slot = slot + 1 == nbuf ? 0 : slot + 1;
    }
  }
}

template <int GM, bool GEN>
__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a) {
  attend_body<GM>(a, [&](const WaveCtx& c, WaveState<GM>& st) { generic_tiles<GM, GEN>(a, c, st); });
}

template <int GM, bool GEN>
static hipError_t launch_gm(const AttendArgs& a, hipStream_t s) {
  const size_t lds = attend_lds_bytes(a.kbuf_words, a.vbuf_words, a.nbuf, a.group) + 4u * a.cb_words;
  const dim3 grid((unsigned)(a.wg_per_row * a.batch));
  hipLaunchKernelGGL((attend_mfma_kernel<GM, GEN>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <bool GEN>
static hipError_t launch_widths(const AttendArgs& a, hipStream_t s) {
  return a.group <= 4 ? launch_gm<4, GEN>(a, s) : a.group <= 8 ? launch_gm<8, GEN>(a, s) : launch_gm<16, GEN>(a, s);
}

// Kernel, tile buffers and resident workgroups per CU for a layout.  The
// specialised kernels fit three waves per SIMD (at most 168 VGPRs), the generic
// ones two; resident workgroups count for more than a third tile buffer (more
// waves hide the LDS and matrix-core latencies of the tile loop).
AttendPlan plan_attend(const HeadTable& heads, int n_kv_heads, int group, bool rope) {
  AttendPlan p;
  int wkm = 1, wvm = 1;
  p.cb_words = 0;
  p.vq = false;
  for (int h = 0; h < n_kv_heads; ++h) {
    const HeadDesc& d = heads.h[h];
    wkm = d.wk > wkm ? d.wk : wkm;
    wvm = d.wv > wvm ? d.wv : wvm;
    p.gen |= !(pow2_bits(d.bk) && pow2_bits(d.bv));
    p.vq |= is_vq(d.bk) || is_vq(d.bv);
    const int cw = vq_lds_words(d.rk, d.bk, d.rv, d.bv);
    p.cb_words = cw > p.cb_words ? cw : p.cb_words;
  }
  p.spec_class = -1;
  if (rope) p.cb_words = rope_lds_words(group <= 4 ? 4 : 8);  // the RoPE kernel: generic tiles and its exchange
  if (group <= 8 && !rope) {
    for (int cls = 0; cls < kSpecClasses + kFrozenClasses && p.spec_class < 0; ++cls) {
      bool all = true;
      for (int h = 0; h < n_kv_heads && all; ++h) {
        const HeadDesc& d = heads.h[h];
        all = class_index(cls, d.rk, d.bk, d.rv, d.bv) >= 0 && d.hk == class_header(cls) && d.hv == class_header(cls);
      }
      if (all) p.spec_class = cls;
    }
  }
  // tile buffers: 64 records plus the 16-byte copy granule and one word read past the last record
  p.kbuf_words = ((64 * wkm + 4 + 3) / 4) * 4;
  p.vbuf_words = ((64 * wvm + 4 + 3) / 4) * 4;
  // LDS per CU, and the hardware's allocation granule (a workgroup's LDS is rounded
  // up to it; 1280 bytes bounds the gfx950 granule from above)
  const size_t kLds = 160 * 1024, kGranule = 1280;
  auto fits = [&](int wpc, int nb) {
    const size_t per_wg =
        (attend_lds_bytes(p.kbuf_words, p.vbuf_words, nb, group) + 4u * p.cb_words + kGranule - 1) / kGranule * kGranule;
    return (size_t)wpc * per_wg <= kLds;
  };
  const int max_wpc = p.spec_class >= 0 ? 3 : 2;
  p.nbuf = 0;
  for (int wpc = max_wpc; wpc >= 1 && p.nbuf == 0; --wpc) {
    for (int nb = 3; nb >= (wpc == 1 ? 1 : 2) && p.nbuf == 0; --nb) {
      if (fits(wpc, nb)) {
        p.nbuf = nb;
        p.wg_per_cu = wpc;
      }
    }
  }
  if (p.nbuf == 0) {  // larger than one CU's LDS at one buffer: not reachable for supported formats
    p.nbuf = 1;
    p.wg_per_cu = 1;
  }
  return p;
}

hipError_t launch_attend(const AttendArgs& a_in, hipStream_t s) {
  if (a_in.rope) return launch_attend_rope(a_in, s);
  AttendArgs a = a_in;
  const AttendPlan p = plan_attend(a.heads, a.n_kv_heads, a.group);
  a.kbuf_words = p.kbuf_words;
  a.vbuf_words = p.vbuf_words;
  a.nbuf = p.nbuf;
  a.cb_words = p.cb_words;
  if (p.vq && p.spec_class < 0) return hipErrorNotSupported;  // the host rejects such layouts first
  if (p.spec_class >= 0) {
    for (int h = 0; h < a.n_kv_heads; ++h) {
      HeadDesc& d = a.heads.h[h];
      d.spec = class_index(p.spec_class, d.rk, d.bk, d.rv, d.bv);
    }
    switch (p.spec_class) {
      case 0: return launch_attend_spec0(a, s);
      case 1: return launch_attend_spec1(a, s);
      case 2: return launch_attend_spec2(a, s);
      case 3: return launch_attend_spec3(a, s);
      case 4: return launch_attend_spec4(a, s);
      case 5: return launch_attend_spec5(a, s);
      case 6: return launch_attend_spec6(a, s);
      default: return launch_attend_frozen(p.spec_class - kSpecClasses, a, s);
    }
  }
  // the generic kernel; all power-of-two widths skip the general-width paths
  return p.gen ? launch_widths<true>(a, s) : launch_widths<false>(a, s);
}

}  // namespace kvtc
