// Split-K decode attention over keys compressed before the rotary position
// embedding (gfx950).
//
// KV-COBRA project page, Results (the note under the results table): the keys are
// compressed before RoPE.  The cache then holds the codes of the unrotated key k_t,
// and the score of token t is q . RoPE(k^_t, t) with k^_t = P_K c^_t: RoPE turns
// every dimension pair (2i, 2i+1) by t theta_i, so the key has to be reconstructed
// in the head dimension and turned by its own position before the dot product (the
// query can no longer be projected once into the key basis, as in the other kernels).
//
// Work split.  The four waves of a workgroup stream their quarters of the split as
// in the other kernels (one 64-token tile per wave and step), but each tile's scores
// are formed by all four: wave w reconstructs dimensions [32w, 32w + 32) of the 64
// tokens of every wave's current tile on the matrix cores, D = P_K(rows) x codes
// (A = the wave's 32 rows of the key basis as fp16 hi + lo, held in registers for the
// whole launch; B = the codes as fp16 subnormals, built as in the score phase of the
// other kernels), adds the header (min * row sum of P_K + step * D), turns each pair
// by its token's position and dots the wave's 32 dimensions with the query, again on
// the matrix cores (the turned key as fp16 hi + lo B operands, the query as the A
// operand with its hi and lo parts in separate rows).  The
// four partial scores of a token meet in LDS and are added in wave order; each wave
// then runs the softmax and the value phase of its own tile exactly as the generic
// kernel does, and the workgroup and split merges are the shared ones.  The matrix
// cores do 2 * 128 * r_K products per token (hi and lo), which at r_K = 128 outweigh
// the record bytes: this kernel is bound by the matrix cores, not by HBM.
//
// Angles.  Lane (n, G) holds token 16 tt + n of each 16-token sub-tile tt of a tile
// that starts at t0: the rotation of its pairs at the first sub-tile, (t0 + n) theta_i,
// comes from a float64 angle reduced modulo 2 pi, once per tile and pair; each later
// sub-tile turns it further by 16 theta_i (angle addition with cos / sin of
// 16 theta_i, fixed per lane).
#include "attend_core.h"

namespace kvtc {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// (cos, sin) of a float64 angle: reduced to [-pi, pi] in float64, then the hardware
// sine and cosine in float32.
__device__ inline void cos_sin(double x, float& c, float& s) {
  const double r = x - kTwoPi * __builtin_rint(x * (1.0 / kTwoPi));
  const float rf = (float)r;
  c = __cosf(rf);
  s = __sinf(rf);
}

// The B operands of one token's codes for the K-steps ks < NKS (lane group G holds the
// pair slots [4 NKS G, 4 NKS (G + 1)) of the token, as in the score phase): rec is the
// token's record shifted so that its codes start at rec[1].
template <int B, int NKS>
__device__ __attribute__((always_inline)) inline void code_operands(const uint32_t* rec, int G, u32x4 (&bop)[NKS]) {
  if constexpr (pow2_bits(B)) {
    constexpr int PPW = Pow2<B>::kPerHalf;
    constexpr int NWL = (NKS * 4 * B + 15) / 16;
    const int base = G * NKS * 4;
    uint32_t w[NWL];
    lds_words<NWL>(rec + 1 + base / PPW, w);
    if constexpr (NKS * 4 < PPW) w[0] >>= (base % PPW) * B;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int pl = ks * 4 + p;
        bop[ks][p] = Pow2<B>::pair(w[pl / PPW], (pl % PPW) * B);
      }
  } else {
    constexpr int SPAN = 8 * NKS * B;
    constexpr int NA = (SPAN + 31) / 32;
    uint32_t a[NA];
    span_words<NA, SPAN % 32 == 0>(rec + 1, G * SPAN, a);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        bop[ks][p] = span_code<B>(a, 8 * ks + 2 * p) | (span_code<B>(a, 8 * ks + 2 * p + 1) << 16);
  }
}

// The wave's key-phase operands.  For the whole launch (registers): its 32 rows of the
// key basis as A operands (rows 16 mb + r16 of the wave's dimensions, pair slots as in
// the score phase) and the scale back from their 2^E.  Reloaded from LDS for each
// source tile (so that they are not live through the softmax and value phases): the
// row sums of its dimensions, cos / sin of 16 theta_i for its pairs, and the query at
// its dimensions as the A operands of the dot product: element j of lane group G is
// dimension 16 (j / 4) + 4 G + j % 4 of the wave's 32 (the dimensions each lane holds
// of a reconstructed key), row = head: aq1 the hi parts in rows [0, GM) and the lo
// parts in rows [GM, 2 GM), aq2 the hi parts alone (for the lo parts of the key).  The
// query carries scale * log2 e * 4 and the key 1 / 4 (headroom below the fp16
// maximum for the key).
struct RopeWave {
  u32x4 ph[2][4], pl[2][4];
  float escale;
};
struct RopeTile {
  float p1[2][4];
  float c16[2][2], s16[2][2];
  u32x4 aq1, aq2;
};

// Partial scores of one source tile (64 tokens at t0): the wave's 32 dimensions of
// each token reconstructed, turned and dotted with the query, added over the lane
// groups and written to out[token][GM].  kt: the tile (records of wk words, header
// first when hk); nvalid tokens are real (the others read stale records: their
// scores are finite and masked by the softmax).
template <int B, int NKS, int GM>
__device__ __attribute__((always_inline)) inline void rope_k_tile(const uint32_t* kt, int wk, int hk, uint32_t skw,
                                                                  const RopeWave& rw, const RopeTile& rt,
                                                                  float (&cr)[2][2], float (&sr)[2][2], float* out) {
  const int lane = threadIdx.x & 63, n = lane & 15, G = lane >> 4;
  const uint32_t* ktc = kt + hk - 1;  // codes of record j start at word j wk + 1
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tok = 16 * tt + n;
    u32x4 bop[NKS];
    code_operands<B, NKS>(ktc + tok * wk, G, bop);
    f32x4 d[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) d[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        d[mb] = mfma(rw.ph[mb][ks], bop[ks], d[mb]);
        d[mb] = mfma(rw.pl[mb][ks], bop[ks], d[mb]);
      }
    const uint32_t kh = hk ? kt[tok * wk] : skw;
    const float mu = f16_bits_to_f32(kh & 0xFFFFu), sg = f16_bits_to_f32(kh >> 16) * rw.escale;
    u32x4 bh, bl;  // the turned key at the lane's 8 dimensions, fp16 hi and lo (times 1/4: the step and
                   // the row sums carry it)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        // this token's key at dimensions 16 mb + 4 G + 2 pp (+1), a pair of the rotation
        const float x = fmaf(sg, d[mb][2 * pp], mu * rt.p1[mb][2 * pp]);
        const float y = fmaf(sg, d[mb][2 * pp + 1], mu * rt.p1[mb][2 * pp + 1]);
        const float c = cr[mb][pp], s = sr[mb][pp];
        const float xr = c * x - s * y, yr = s * x + c * y;
        if (tt < 3) {  // on to the token 16 positions later
          cr[mb][pp] = c * rt.c16[mb][pp] - s * rt.s16[mb][pp];
          sr[mb][pp] = s * rt.c16[mb][pp] + c * rt.s16[mb][pp];
        }
        // hi = the pair truncated to fp16 (packed conversion), lo = the exact remainder
        // truncated again: ~21 significant bits
        const auto hp = __builtin_amdgcn_cvt_pkrtz(xr, yr);
        const auto lp = __builtin_amdgcn_cvt_pkrtz(xr - (float)hp[0], yr - (float)hp[1]);
        bh[2 * mb + pp] = __builtin_bit_cast(uint32_t, hp);
        bl[2 * mb + pp] = __builtin_bit_cast(uint32_t, lp);
      }
    }
    // rows [0, GM): hi(q) . (hi(k) + lo(k)); rows [GM, 2 GM): lo(q) . hi(k)
    f32x4 sc = mfma(rt.aq1, bh, f32x4{0.f, 0.f, 0.f, 0.f});
    sc = mfma(rt.aq2, bl, sc);
    // lane group G holds rows 4G .. 4G+3: add the lo rows to the hi rows of the same heads
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] += __shfl_xor(sc[e], GM == 4 ? 16 : 32);
    if (4 * G < GM) *(f32x4*)(out + tok * GM + 4 * G) = sc;
    __builtin_amdgcn_sched_barrier(0);  // one sub-tile's operands live at a time (registers)
  }
}

#define KVTC_ROPE_K(B)                                                            \
  case B:                                                                         \
    if (nks == 1) rope_k_tile<B, 1, GM>(kt, wk, hk, skw, rw, rt, cr, sr, out);        \
    else if (nks == 2) rope_k_tile<B, 2, GM>(kt, wk, hk, skw, rw, rt, cr, sr, out);   \
    else rope_k_tile<B, 4, GM>(kt, wk, hk, skw, rw, rt, cr, sr, out);                 \
    break;
#define KVTC_ROPE_V(B)                                                                       \
  case B:                                                                                    \
    if (NT == 1) v_phase<B, 1, true>(vtc, wv, kk, ahi, alo, st.acc2);                        \
    else if (NT == 2) v_phase<B, 2, true>(vtc, wv, kk, ahi, alo, st.acc2);                   \
    else if (NT == 4) v_phase<B, 4, true>(vtc, wv, kk, ahi, alo, st.acc2);                   \
    else v_phase<B, 8, true>(vtc, wv, kk, ahi, alo, st.acc2);                                \
    break;

// The tile loop of the RoPE kernel.  All four waves take the same number of steps
// (a split's waves stream equal numbers of 64-token tiles, empty past the context)
// and meet at two barriers per step: once every wave's tile is in LDS, and once the
// partial scores are.
template <int GM>
__device__ __attribute__((always_inline)) inline void rope_tiles(const AttendArgs& a, const WaveCtx& c,
                                                                 WaveState<GM>& st) {
  const HeadDesc hd = head_desc(a.heads, c.h);
  const int rk = __builtin_amdgcn_readfirstlane(hd.rk), rv = __builtin_amdgcn_readfirstlane(hd.rv);
  const int bk = __builtin_amdgcn_readfirstlane(hd.bk), bv = __builtin_amdgcn_readfirstlane(hd.bv);
  const int wk = hd.wk, wv = hd.wv;
  const int hk = __builtin_amdgcn_readfirstlane(hd.hk), hv = __builtin_amdgcn_readfirstlane(hd.hv);
  const uint32_t skw = __builtin_amdgcn_readfirstlane(hd.sk), svw = __builtin_amdgcn_readfirstlane(hd.sv);
  const int nks = rk >= 32 ? rk / 32 : 1;
  const int NT = rv / 16;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, G = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbuf = c.nbuf, g = c.g;
  const float* P = a.basis_k + hd.qoff_k;  // keys are reconstructed through the query-side basis
  float* part = c.extra;                   // [src wave][tile wave][64][GM]
  float* p1s = c.extra + kWaves * kWaves * kTileT * GM;  // [128] row sums
  float* cs16 = p1s + kHeadDim;                          // [64][2] cos, sin of 16 theta_i
  double* ths = (double*)(cs16 + kHeadDim);              // [64] inverse frequencies
  uint32_t* aqs = (uint32_t*)(ths + kHeadDim / 2);       // [wave][lane][8] query operands
  const uint32_t kl = lds_addr(c.ktile), vl = lds_addr(c.vtile);
  const int64_t bq0 = (int64_t)c.b * a.n_q_heads + (int64_t)c.h * g;

  // ---- the wave's registers: basis rows as A operands (with their exponent), the
  // query at its dimensions, the row sums, the per-slot rotations
  RopeWave rw;
  {
    float pv[2][4][4][2];
    int sh[4][4];
    float mx = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        bool valid = false;
        int jl = 0, jh = 0, s = 0;
        if (ks < nks) k_slot_rt(bk, G, nks, ks, p, rk, valid, jl, jh, s);
        sh[ks][p] = s;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const float* row = P + (int64_t)(32 * wave + 16 * mb + n) * rk;
          const float xl = valid && ks < nks ? row[jl] : 0.0f, xh = valid && ks < nks ? row[jh] : 0.0f;
          pv[mb][ks][p][0] = xl;
          pv[mb][ks][p][1] = xh;
          mx = fmaxf(mx, fmaxf(fabsf(xl), fabsf(xh)));
        }
      }
    mx = wave_max(mx);
    int e = 0;
    if (mx > 0.0f) {
      frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
      e = 14 - e;      // max |P| 2^E < 2^14
    }
    rw.escale = ldexpf(1.0f, 22 - e);  // codes are fp16 subnormals (code 2^-24); the key carries 1/4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float xl = ldexpf(pv[mb][ks][p][0], e - sh[ks][p]), xh = ldexpf(pv[mb][ks][p][1], e - sh[ks][p]);
          const _Float16 hl = (_Float16)xl, hh = (_Float16)xh;
          const _Float16 ll = (_Float16)(xl - (float)hl), lh = (_Float16)(xh - (float)hh);
          rw.ph[mb][ks][p] = h2u(hl) | (h2u(hh) << 16);
          rw.pl[mb][ks][p] = h2u(ll) | (h2u(lh) << 16);
        }
  }
  {
    // the query operands: row r16 of lane group G, element j = dimension
    // 32 wave + 16 (j / 4) + 4 G + j % 4
    const int row = n, head = row % GM;
    const bool on = row < 2 * GM && head < g;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t w1 = 0u, w2 = 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 2 * p + u;
        const int dim = 32 * wave + 16 * (j >> 2) + 4 * G + (j & 3);
        float qv = 0.0f;
        if (on) {
          const int64_t off = (bq0 + head) * kHeadDim + dim;
          qv = (a.dtype == 0 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off]) * a.scale_log2 * 4.0f;
        }
        const _Float16 qh = (_Float16)qv, ql = (_Float16)(qv - (float)qh);
        w1 |= h2u(row < GM ? qh : ql) << (16 * u);
        w2 |= h2u(row < GM ? qh : (_Float16)0.0f) << (16 * u);
      }
      aqs[(wave * 64 + lane) * 8 + p] = w1;
      aqs[(wave * 64 + lane) * 8 + 4 + p] = w2;
    }
  }
  // row sums of the basis, two threads per row (in order within each half row)
  {
    const int row = tid >> 1, half = tid & 1, hr = rk / 2;
    const float* pr = P + (int64_t)row * rk + half * hr;
    float sum = 0.0f;
    for (int j = 0; j < hr; ++j) sum += pr[j];
    sum += __shfl_xor(sum, 1);
    if (half == 0) p1s[row] = sum * 0.25f;  // the key carries 1/4
  }
  // the first tiles, behind the loads above
  for (int t = 0; t < (nbuf > 1 ? nbuf - 1 : 1); ++t) {
    const int t0 = c.t_begin + t * kTileT;
    if (t0 < c.t_end) {
      const int nn = (c.t_end - t0) < kTileT ? (c.t_end - t0) : kTileT;
      const uint32_t r0 = tile_rec(c, t0);
      tile_copy(c.rk_, r0 * 4u * wk, (uint32_t)nn * 4u * wk, kl + 4u * (uint32_t)(t * c.kbuf));
      tile_copy(c.rv_, r0 * 4u * wv, (uint32_t)nn * 4u * wv, vl + 4u * (uint32_t)(t * c.vbuf));
    }
  }
  if (tid < kHeadDim / 2) {  // frequencies and the turn of 16 positions, per pair
    const double th = a.rope[tid];
    ths[tid] = th;
    cos_sin(16.0 * th, cs16[2 * tid], cs16[2 * tid + 1]);
  }
  __syncthreads();  // row sums, frequencies, turns and query operands in LDS
  if (threadIdx.x == 0) KVTC_STAMP(c.stamp, 1);

  init_state(st);
  float* S = c.S;
  if (lane < 4) ((uint32_t*)S)[score_floats(GM) + lane] = 0u;  // zero slot
  float sq[GM], kf[GM];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    sq[hh] = 0.0f;  // the scores arrive final: s = 1 * 1 * S + 0
    kf[hh] = 1.0f;
  }
  constexpr uint32_t kUnitStep = 0x3C00u << 16;  // fp16 min 0, step 1
  const int steps = c.wave_tokens / kTileT;
  int slot = 0;
  for (int k = 0; k < steps; ++k) {
    wait_tiles();     // this wave's tile of step k
    __syncthreads();  // every wave's tile of step k is in LDS, and every wave is done with step k - 1
    const int t0w = c.t_begin + k * kTileT;
    if (nbuf >= 2) {
      const int tn = t0w + (nbuf - 1) * kTileT;
      if (tn < c.t_end) {
        const int nn = (c.t_end - tn) < kTileT ? (c.t_end - tn) : kTileT;
        int sn = slot + nbuf - 1;
        sn = sn >= nbuf ? sn - nbuf : sn;
        const uint32_t rn = tile_rec(c, tn);
        tile_copy(c.rk_, rn * 4u * wk, (uint32_t)nn * 4u * wk, c.ktile + sn * c.kbuf);
        tile_copy(c.rv_, rn * 4u * wv, (uint32_t)nn * 4u * wv, c.vtile + sn * c.vbuf);
      }
    }
    // ---- partial scores of the four waves' tiles at this wave's dimensions
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const int tb = c.split_begin + w2 * c.wave_tokens, t0 = tb + k * kTileT;
      const int te = tb + c.wave_tokens < c.n_tok ? tb + c.wave_tokens : c.n_tok;
      if (t0 >= te) continue;  // uniform: that wave's tile is past the context
      const uint32_t* kt = c.ktile + (w2 - wave) * c.wave_area + slot * c.kbuf;
      RopeTile rt;
      float cr[2][2], sr[2][2];  // this lane's token of the first sub-tile, t0 + n
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int i0 = 16 * wave + 8 * mb + 2 * G;  // the lane's first pair of this row block
        *(f32x4*)rt.p1[mb] = *(const f32x4*)(p1s + 2 * i0);
        const f32x4 cs = *(const f32x4*)(cs16 + 2 * i0);
        rt.c16[mb][0] = cs[0];
        rt.s16[mb][0] = cs[1];
        rt.c16[mb][1] = cs[2];
        rt.s16[mb][1] = cs[3];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) cos_sin((double)(t0 + n) * ths[i0 + pp], cr[mb][pp], sr[mb][pp]);
      }
      rt.aq1 = *(const u32x4*)(aqs + (wave * 64 + lane) * 8);
      rt.aq2 = *(const u32x4*)(aqs + (wave * 64 + lane) * 8 + 4);
      float* out = part + (wave * kWaves + w2) * kTileT * GM;
      switch (bk) { KVTC_ROPE_K(2) KVTC_ROPE_K(3) KVTC_ROPE_K(4) KVTC_ROPE_K(5) KVTC_ROPE_K(6) KVTC_ROPE_K(7) KVTC_ROPE_K(8) }
    }
    __syncthreads();  // partial scores complete
    const int nvalid = c.t_end - t0w < kTileT ? c.t_end - t0w : kTileT;
    if (nvalid > 0) {
      const uint32_t* kt = c.ktile + slot * c.kbuf;
      const uint32_t* vt = c.vtile + slot * c.vbuf;
      const uint32_t* vtc = vt + hv - 1;
      // this tile's scores: the four partials added in wave order, S as the softmax reads it
#pragma unroll
      for (int q4 = 0; q4 < GM / 4; ++q4) {
        f32x4 sc = *(const f32x4*)(part + (0 * kWaves + wave) * kTileT * GM + lane * GM + 4 * q4);
#pragma unroll
        for (int w2 = 1; w2 < kWaves; ++w2) sc += *(const f32x4*)(part + (w2 * kWaves + wave) * kTileT * GM + lane * GM + 4 * q4);
        if constexpr (kpack(GM)) {
          *(f32x4*)(S + lane * 2 * GM + 4 * q4) = sc;
          *(f32x4*)(S + lane * 2 * GM + GM + 4 * q4) = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
          *(f32x4*)(S + lane * GM + 4 * q4) = sc;
        }
      }
      lds_fence();
      softmax_tile<GM>(kt, vt, wk, wv, 0, hv, kUnitStep, svw, nvalid, g, S, sq, kf, st);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 ahi, alo;
        p_operands<GM>(S, kk, ahi, alo);
        switch (bv) { KVTC_ROPE_V(2) KVTC_ROPE_V(3) KVTC_ROPE_V(4) KVTC_ROPE_V(5) KVTC_ROPE_V(6) KVTC_ROPE_V(7) KVTC_ROPE_V(8) }
      }
      lds_fence();
    }
    if (nbuf == 1) {
      __syncthreads();  // every wave is done with this step's tiles
      const int t1 = t0w + kTileT;
      if (t1 < c.t_end) {
        const int n1 = (c.t_end - t1) < kTileT ? (c.t_end - t1) : kTileT;
        const uint32_t r1 = tile_rec(c, t1);
        tile_copy(c.rk_, r1 * 4u * wk, (uint32_t)n1 * 4u * wk, c.ktile);
        tile_copy(c.rv_, r1 * 4u * wv, (uint32_t)n1 * 4u * wv, c.vtile);
      }
    } else {
      slot = slot + 1 == nbuf ? 0 : slot + 1;
    }
  }
}

template <int GM>
__global__ __launch_bounds__(256, 2) void attend_rope_kernel(AttendArgs a) {
  attend_body<GM>(a, [&](const WaveCtx& c, WaveState<GM>& st) { rope_tiles<GM>(a, c, st); });
}

}  // namespace

hipError_t launch_attend_rope(const AttendArgs& a_in, hipStream_t s) {
  AttendArgs a = a_in;
  if (a.group > 8) return hipErrorNotSupported;  // the host rejects such layouts first
  const AttendPlan p = plan_attend(a.heads, a.n_kv_heads, a.group, true);
  if (p.vq) return hipErrorNotSupported;
  a.kbuf_words = p.kbuf_words;
  a.vbuf_words = p.vbuf_words;
  a.nbuf = p.nbuf;
  a.cb_words = p.cb_words;
  const size_t lds = attend_lds_bytes(a.kbuf_words, a.vbuf_words, a.nbuf, a.group) + 4u * a.cb_words;
  const dim3 grid((unsigned)(a.wg_per_row * a.batch));
  if (a.group <= 4) hipLaunchKernelGGL((attend_rope_kernel<4>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((attend_rope_kernel<8>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace kvtc
