// a2: weighted-ReLU block scores on MFMA.
//
// CSA page (nemo_automodel...step5.sparse), indexer_score_tile: one bounded
// FP32 tile of scores sum_h w[t,h] * relu(q[t,h] . k[j]) with signed FP32
// head weights; visibility and scale per the QSA page, select_qsa_token_ids.
//
// Tiling.  Rows of the MFMA A operand are (query, head) pairs, columns are
// blocks, K is the index dimension.  A workgroup (4 waves) owns the rows of
// 4 * 16 RT / H queries -- each wave keeps RT row tiles (whole queries) of q in
// registers for the whole launch -- and the whole visible block range of those
// queries.  It streams the range in chunks of blocks: the FP32 compressed keys are split into
// bf16 high and low halves on the way into a double-buffered LDS tile, and
// every wave reads each 16-block operand once for all of its row tiles
// (q*hi + q*lo, plus q_lo*hi for FP32 queries).  The accumulator layout puts
// 4 heads of one query in each lane, so the weighted head reduction is in-lane
// FMAs plus at most two cross-lane adds.
#include <algorithm>

#include "irb_internal.hpp"

namespace irb {

constexpr int kScoreChunk = 64;   // blocks per LDS chunk

template <typename QT>
IRB_DEV void load_q_operand(const QT* p, bf16x8& hi, bf16x8& lo);

template <>
IRB_DEV void load_q_operand<uint16_t>(const uint16_t* p, bf16x8& hi, bf16x8& lo) {
  hi = *reinterpret_cast<const bf16x8*>(p);
  (void)lo;
}

template <>
IRB_DEV void load_q_operand<float>(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t h, l;
    split_bf16(f[e], h, l);
    hi[e] = static_cast<short>(h);
    lo[e] = static_cast<short>(l);
  }
}

// Index-query preparation fused into the q loads (QSA page: the indexer's
// q_layernorm and apply_qsa_rope, consumed by select_qsa_token_ids).  This
// lane holds dimensions 32 s + 8 g16 + e (s < D / 32, e < 8) of its row; the
// four lanes g16 = 0..3 of a row together hold all of it.  The arithmetic
// is that of the preparation kernel step for step, so the operands equal
// the prepared queries exactly: per-chunk sums of squares (that kernel's
// chunks of EPL dimensions, fmas in dimension order), the same pairwise
// tree over chunks (a chunk pairs with chunk ^ o, o = chunks / 2 .. 1), the
// same reciprocal square root, gain and fma rotation, one rounding to QT.
// The rotation partner d +- R / 2 of a dimension sits in this lane's own
// registers because R / 2 is a multiple of 32.
template <typename QT, int D>
IRB_DEV void prep_q_operands(const QT* qp, const float* rope_row, int g16, const QPrep& pp, const float (&gm)[D / 32][8],
                             bf16x8 (&qh)[D / 32], bf16x8 (&ql)[D / 32]) {
  constexpr int KS = D / 32;
  constexpr int EPL = sizeof(QT) == 2 ? 8 : 4;   // the preparation kernel's dimensions per lane (D <= 128)
  constexpr int HPL = 8 / EPL;                   // its chunks per run of 8 dimensions here
  constexpr int LPR = D / EPL;                   // its chunks per row
  const int R = pp.R, half = R / 2;
  // full-width rotation (the usual case): run s pairs with run s ^ (KS / 2)
  // and both use the same table entries
  const bool full = R == D;
  // every load first (raw row, rotary factors), so their latencies overlap;
  // runs past R read the gain row instead (a valid address) and discard it
  float x[KS][8], cs[KS][8], sn[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if constexpr (sizeof(QT) == 2) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = bf16_to_f32(static_cast<uint16_t>(v[e]));
    } else {
      const float4 a = *reinterpret_cast<const float4*>(qp + 32 * s);
      const float4 c = *reinterpret_cast<const float4*>(qp + 32 * s + 4);
      x[s][0] = a.x; x[s][1] = a.y; x[s][2] = a.z; x[s][3] = a.w;
      x[s][4] = c.x; x[s][5] = c.y; x[s][6] = c.z; x[s][7] = c.w;
    }
  }
  if (full) {
#pragma unroll
    for (int s = 0; s < (KS > 1 ? KS / 2 : 1); ++s) {
      const int j0 = 32 * s + 8 * g16;
      const float4 c0 = *reinterpret_cast<const float4*>(rope_row + j0);
      const float4 c1 = *reinterpret_cast<const float4*>(rope_row + j0 + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(rope_row + half + j0);
      const float4 s1 = *reinterpret_cast<const float4*>(rope_row + half + j0 + 4);
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[s][e] = cv[e];
        sn[s][e] = -sv[e];
        if (KS > 1) {
          cs[(s + KS / 2) % KS][e] = cv[e];
          sn[(s + KS / 2) % KS][e] = sv[e];
        }
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d0 = 32 * s + 8 * g16;
      const bool rot = d0 < R;
      const int j0 = d0 < half ? d0 : d0 - half;
      const float* cp = rot ? rope_row + j0 : pp.gamma;
      const float* sp = rot ? rope_row + half + j0 : pp.gamma;
      const float4 c0 = *reinterpret_cast<const float4*>(cp), c1 = *reinterpret_cast<const float4*>(cp + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(sp), s1 = *reinterpret_cast<const float4*>(sp + 4);
      const float sg = d0 < half ? -1.f : 1.f;
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[s][e] = rot ? cv[e] : 1.f;
        sn[s][e] = rot ? sg * sv[e] : 0.f;
      }
    }
  }
  // chunk (s, h) is the preparation kernel's chunk (4 s + g16) HPL + h
  float p[KS][HPL];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int h = 0; h < HPL; ++h) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(x[s][h * EPL + e], x[s][h * EPL + e], a);
      p[s][h] = a;
    }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) {
    if (o < HPL) {                               // the other half of this lane's run
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float a = p[s][0], c = p[s][HPL - 1];
        p[s][0] = a + c;
        p[s][HPL - 1] = c + a;
      }
    } else if (o < 4 * HPL) {                    // the same run in lane group g16 ^ (o / HPL)
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h = 0; h < HPL; ++h) p[s][h] += __shfl_xor(p[s][h], 16 * (o / HPL), 64);
    } else {                                     // run s ^ (o / (4 HPL)) of this lane
      float n[KS][HPL];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h = 0; h < HPL; ++h) n[s][h] = p[s][h] + p[s ^ (o / (4 * HPL))][h];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h = 0; h < HPL; ++h) p[s][h] = n[s][h];
    }
  }
  const float inv = 1.0f / sqrtf(p[0][0] / static_cast<float>(D) + pp.eps);
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[s][e] = x[s][e] * inv * gm[s][e];
  // the partner of run s: run s ^ (KS / 2) for a full-width rotation, else picked at run time
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int d0 = 32 * s + 8 * g16;
    // the rotation partner run (itself past R, where the sine factor is 0)
    const int ps = d0 < half ? s + half / 32 : (d0 < R ? s - half / 32 : s);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float pv = x[KS > 1 ? s ^ (KS / 2) : s][e];
      if (!full) {
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) pv = s2 == ps ? x[s2][e] : pv;
      }
      const float y = fmaf(x[s][e], cs[s][e], pv * sn[s][e]);
      if constexpr (sizeof(QT) == 2) {
        qh[s][e] = static_cast<short>(f32_to_bf16(y));
      } else {
        uint16_t h, l;
        split_bf16(y, h, l);
        qh[s][e] = static_cast<short>(h);
        ql[s][e] = static_cast<short>(l);
      }
    }
  }
}

// gamma and the rotary rows are read 16 bytes at a time (16-byte aligned)
bool score_prep_ok(int D, int R) { return R == 0 || (R > 0 && R % 64 == 0 && R <= D); }

// Row tiles (16 rows each) of q held per wave, always whole queries.  FP32
// queries (hi/lo operands) and 4-head queries keep two at D = 128 so that
// their operands fit in registers.  (Eight row tiles halve the LDS key reads
// per MFMA but halve the number of workgroups, which measured slower.)
template <typename QT, int D, int H, bool kPre>
constexpr int score_rt() {
  if (sizeof(QT) == 4 || H <= 4) return (D == 128 && H <= 32) ? 2 : ((64 % H == 0) ? 4 : 3);
  return (64 % H == 0) ? 4 : 3;
}

// Visible block range of query t: [base, base + nb) (nb = 0 when not valid)
IRB_DEV void visible_blocks(const Layout& L, const int32_t* cu_blocks, int c, int b, int t, int& base, int& nb) {
  const Doc d = doc_of(L, b, t);
  base = d.valid ? block_base(L, cu_blocks, d) : 0;
  nb = d.valid ? (t - d.start + 1) / c : 0;
}

// kPre: the keys come pre-split (kcs, per block a row of bf16 high halves then
// a row of low halves) and stream through four LDS buffers by direct
// global-to-LDS loads, three chunks in flight; otherwise the FP32 keys are
// split while staging through two buffers.
// GS = 4 or 8 (with H a multiple of 16): the H heads are H / GS groups of GS
// heads with one score each ([CSA] indexer_score_tile, scores per KV group),
// all groups in one launch.  The four accumulator rows a lane holds are
// heads 4 g16 .. 4 g16 + 3 of its row tile: for GS = 4 exactly one group,
// so each lane's weighted sum is that group's score; for GS = 8 one pair
// exchange between lane groups (g16, g16 ^ 1) completes it.  Group gi's
// tile starts gi * gstride floats after out.  GS = 0: one score per query
// over all H heads.
template <typename QT, int D, int H, bool kPre, int GS>
__global__ void __launch_bounds__(256, 2)
score_kernel(Layout L, const QT* __restrict__ q, const float* __restrict__ w, const float* __restrict__ kc,
             const uint16_t* __restrict__ kcs, const int32_t* __restrict__ cu_blocks, int c, float scale, int q0,
             int q1, int j0, int j1, float* __restrict__ out, int64_t ostride, int seg_blocks, int n_seg,
             int write_invisible, int skip_nb, int n_grp, int64_t gstride, QPrep prep) {
  static_assert(GS == 0 || ((GS == 4 || GS == 8) && H % 16 == 0), "grouped scores: groups of 4 or 8 heads, H a multiple of 16");
  constexpr int NGRP = GS ? H / GS : 1;             // score tiles written
  constexpr bool kPerQ = H < 16 || GS > 0;          // visible ranges kept per query (wave-uniform)
  constexpr int KS = D / 32;
  constexpr bool kSplitQ = sizeof(QT) == 4;
  // row tiles per wave (whole queries); FP32 queries (hi/lo operands) and
  // 4-head queries (16 per wave) keep half as many at D = 128 to stay in registers
  constexpr int RT = score_rt<QT, D, H, kPre>();
  constexpr int QW = 16 * RT / H;                   // queries per wave (>= 1)
  constexpr int QG = 4 * QW;                        // queries per workgroup
  constexpr int LDK = D + 8;                        // padded LDS row (bf16 elements)
  constexpr int CH = kPre ? 32 : kScoreChunk;       // blocks per chunk
  constexpr int NBUF = kPre ? 4 : 2;
  constexpr int GROUPS = kScoreChunk * D / 8;       // 8-dim groups per chunk (split staging)
  constexpr int GPT = GROUPS / 256;                 // per thread
  static_assert(GROUPS % 256 == 0, "chunk staging");
  constexpr int NC = D / 8;                         // 16-byte chunks per bf16 row
  constexpr int PBUF = CH * 2 * D * 2;              // bytes per pre-split buffer
  constexpr int NI = CH * 2 * NC / 256;             // direct loads per wave per chunk
  static_assert(!kPre || NI >= 1, "pre-split staging");
  constexpr int RAW = kPre ? NBUF * PBUF : 2 * 2 * kScoreChunk * LDK * 2;
  __shared__ __align__(16) char kraw[RAW];
  __shared__ int s_range[2];
  __shared__ int s_vis[2][64];          // visible block range (base, nb) of each query

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int b = blockIdx.y;
  // query groups run latest (longest visible range) first
  const int qg = (gridDim.x / n_seg - 1) - blockIdx.x / n_seg, sg = blockIdx.x % n_seg;
  const int qa = q0 + qg * QG, qe = min(q1, qa + QG);
  const int nb_max = L.S / c;

  // visible block range of the workgroup's queries, clipped to [j0, j1) and the segment
  if (tid < 64) {
    int lo = 0x7fffffff, hi = -1;
    int base = 0, nb = 0;
    if (tid < QG && qa + tid < qe) {
      visible_blocks(L, cu_blocks, c, b, qa + tid, base, nb);
      if (nb > skip_nb && nb > 0) { lo = base; hi = base + nb; }
    }
    if (tid < QG) { s_vis[0][tid] = base; s_vis[1][tid] = nb; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o, 64));
      hi = max(hi, __shfl_xor(hi, o, 64));
    }
    if (tid == 0) { s_range[0] = lo; s_range[1] = hi; }
  }
  __syncthreads();
  const int sb = j0 + sg * seg_blocks, se = min(j1, sb + seg_blocks);   // this segment
  const int cb = max(sb, s_range[0]), ce = min(se, s_range[1]);        // computed blocks
  float* otile = out + (static_cast<int64_t>(b) * (q1 - q0) + (qa - q0)) * ostride;
  if (write_invisible) {
    // -inf for the segment's blocks outside [cb, ce) (the computed ones are written below)
    for (int gi = 0; gi < NGRP; ++gi)
      for (int i = tid; i < (qe - qa) * (se - sb); i += 256) {
        const int r = i / (se - sb), j = sb + i % (se - sb);
        if (j < cb || j >= ce) otile[gi * gstride + static_cast<int64_t>(r) * ostride + (j - j0)] = -INFINITY;
      }
  }
  if (cb >= ce) return;

  // pre-split chunk loader: lane i of load n fills 16-byte slot (w NI + n) 64 + i;
  // row R = 2 block + (0 hi | 1 lo), chunk slot sc holds chunk sc ^ ((R / 2) mod NC).
  // The chunk's first block gives a wave-uniform base address (scalar
  // registers); the per-lane byte offsets from it are fixed for the whole
  // launch, and only a chunk reaching past the last block clamps its rows.
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  uint32_t poff[kPre ? NI : 1];
  if constexpr (kPre) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int slot = (wu * NI + n) * 64 + lane;
      const int R = slot / NC, sc = slot % NC;
      poff[n] = static_cast<uint32_t>(R * D + 8 * (sc ^ ((R >> 1) & (NC - 1)))) * 2u;
    }
  }
  const uint32_t klds = lds_addr(kraw);
  auto issue = [&](int j, int pbuf) __attribute__((always_inline)) {
    j = __builtin_amdgcn_readfirstlane(j);
    pbuf = __builtin_amdgcn_readfirstlane(pbuf);
    const uint32_t lb = klds + pbuf * PBUF + wu * NI * 1024;
    if (j + CH <= nb_max) {
      const uint16_t* sb = kcs + (static_cast<int64_t>(b) * nb_max + j) * 2 * D;
#pragma unroll
      for (int n = 0; n < NI; ++n) lds_dma16_s(sb, poff[n], lb + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int slot = (wu * NI + n) * 64 + lane;
        const int R = slot / NC, sc = slot % NC;
        const int blk = min(j + (R >> 1), nb_max - 1);
        const uint16_t* src = kcs + ((static_cast<int64_t>(b) * nb_max + blk) * 2 + (R & 1)) * D +
                              8 * (sc ^ ((R >> 1) & (NC - 1)));
        lds_dma16(src, lb + n * 1024);
      }
    }
  };
  // the first chunks' loads go out before the q rows are loaded (and prepared)
  const int nch = (ce - cb + CH - 1) / CH;
  if constexpr (kPre) {
    for (int p = 0; p < NBUF - 1 && p < nch; ++p) issue(cb + p * CH, p);
  }

  // q rows of this wave in the A layout: row 16 rt + l16 -> query rr / H, head rr % H
  bf16x8 qh[RT][KS], ql[RT][KS];
  float wv[RT][4];
  // q rows and weights are [.., S, n_grp, H, ..]: q and w point at this
  // call's group, one token holds n_grp groups of H heads (1: no group axis)
  const int64_t qrow = static_cast<int64_t>(n_grp) * H * D;
  // gain of this lane's dimensions (fused preparation only)
  float gm[KS][8];
  if (prep.gamma) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4 g0 = *reinterpret_cast<const float4*>(prep.gamma + 32 * s + 8 * g16);
      const float4 g1 = *reinterpret_cast<const float4*>(prep.gamma + 32 * s + 8 * g16 + 4);
      gm[s][0] = g0.x; gm[s][1] = g0.y; gm[s][2] = g0.z; gm[s][3] = g0.w;
      gm[s][4] = g1.x; gm[s][5] = g1.y; gm[s][6] = g1.z; gm[s][7] = g1.w;
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = 16 * rt + l16;
    const int qi = qa + wid * QW + rr / H, hd = rr % H;
    const bool ok = qi < qe;
    const int64_t tok = static_cast<int64_t>(b) * L.S + (ok ? qi : qa);
    const QT* qp = q + tok * qrow + static_cast<int64_t>(hd) * D + 8 * g16;
    if (prep.gamma) {
      prep_q_operands<QT, D>(qp, prep.rope + tok * prep.R, g16, prep, gm, qh[rt], ql[rt]);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) load_q_operand<QT>(qp + 32 * s, qh[rt][s], ql[rt][s]);
    }
    if (!ok) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) { qh[rt][s][e] = 0; if (kSplitQ) ql[rt][s][e] = 0; }
    }
    // head weights of this lane's accumulator rows 16 rt + 4 g16 + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r2 = 16 * rt + 4 * g16 + i;
      const int qw = qa + wid * QW + r2 / H;
      wv[rt][i] = qw < qe ? w[(static_cast<int64_t>(b) * L.S + qw) * (n_grp * H) + r2 % H] : 0.f;
    }
  }

  // chunk staging: thread owns GPT groups of 8 dims (block = grp / (D/8))
  const float* kcb = kc + static_cast<int64_t>(b) * nb_max * D;
  float4 stg[GPT][2];
  auto gload = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int grp = tid + 256 * u;
      const int r = grp / (D / 8), c8 = grp % (D / 8);
      const int jj = min(j + r, nb_max - 1);
      const float* src = kcb + static_cast<int64_t>(jj) * D + 8 * c8;
      stg[u][0] = *reinterpret_cast<const float4*>(src);
      stg[u][1] = *reinterpret_cast<const float4*>(src + 4);
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int grp = tid + 256 * u;
      const int r = grp / (D / 8), c8 = grp % (D / 8);
      const float f[8] = {stg[u][0].x, stg[u][0].y, stg[u][0].z, stg[u][0].w,
                          stg[u][1].x, stg[u][1].y, stg[u][1].z, stg[u][1].w};
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t h, l;
        split_bf16(f[e], h, l);
        hi[e] = static_cast<short>(h);
        lo[e] = static_cast<short>(l);
      }
      uint16_t* kb = reinterpret_cast<uint16_t*>(kraw) + buf * 2 * kScoreChunk * LDK;
      *reinterpret_cast<bf16x8*>(&kb[r * LDK + 8 * c8]) = hi;
      *reinterpret_cast<bf16x8*>(&kb[kScoreChunk * LDK + r * LDK + 8 * c8]) = lo;
    }
  };

  // visible ranges of the wave's queries in registers (the stores test them every tile)
  int my_vb = 0, my_vn = 0;
  bool my_q = false;
  int64_t my_off = 0;
  int vbk[kPerQ ? QW : 1], vnk[kPerQ ? QW : 1];
  if constexpr (!kPerQ) {
    const int k = g16 < QW ? g16 : 0;
    my_vb = s_vis[0][wid * QW + k];
    my_vn = s_vis[1][wid * QW + k];
    my_q = g16 < QW && qa + wid * QW + g16 < qe;
    my_off = static_cast<int64_t>(wid * QW + k) * ostride;
  } else {
#pragma unroll
    for (int k = 0; k < QW; ++k) {
      vbk[k] = __builtin_amdgcn_readfirstlane(s_vis[0][wid * QW + k]);
      vnk[k] = __builtin_amdgcn_readfirstlane(s_vis[1][wid * QW + k]);
    }
  }
  if constexpr (!kPre) {
    gload(cb);
    lstore(0);
    __syncthreads();
  }
  for (int it = 0; it < nch; ++it) {
    const int j = cb + it * CH;
    const int buf = it % NBUF;
    if constexpr (kPre) {
      // this wave's loads of chunk it are done once at most the later chunks'
      // loads (and any score stores issued after them) are outstanding
      const int ahead = min(NBUF - 2, nch - 1 - it);
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(kDmaWait<2 * NI>());
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(kDmaWait<NI>());
      else __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
      bare_barrier();
      if (it + NBUF - 1 < nch) issue(cb + (it + NBUF - 1) * CH, (it + NBUF - 1) % NBUF);
    } else {
      if (it + 1 < nch) gload(j + CH);
    }
    // key operands of column tile ct (16 blocks) from the chunk buffer into slot ct % 2
    bf16x8 okh[2][KS], okl[2][KS];
    auto ld_ops = [&](int ct) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (kPre) {
          const int R = 2 * (16 * ct + l16);
          const int sl = (4 * s + g16) ^ ((R >> 1) & (NC - 1));
          const char* base = kraw + buf * PBUF;
          okh[ct & 1][s] = *reinterpret_cast<const bf16x8*>(base + (R * NC + sl) * 16);
          okl[ct & 1][s] = *reinterpret_cast<const bf16x8*>(base + ((R + 1) * NC + sl) * 16);
        } else {
          const uint16_t* kb = reinterpret_cast<const uint16_t*>(kraw) + buf * 2 * kScoreChunk * LDK;
          const int off = (16 * ct + l16) * LDK + 32 * s + 8 * g16;
          okh[ct & 1][s] = *reinterpret_cast<const bf16x8*>(&kb[off]);
          okl[ct & 1][s] = *reinterpret_cast<const bf16x8*>(&kb[kScoreChunk * LDK + off]);
        }
      }
    };
    ld_ops(0);
#pragma unroll
    for (int ct = 0; ct < CH / 16; ++ct) {
      const int jc = j + 16 * ct;                  // first block of this column tile
      if (jc >= ce) break;
      // the next tile's operands load while this tile's MFMAs and epilogue run
      // (rows of the chunk buffer past ce hold stale keys and are never used)
      if (ct + 1 < CH / 16) ld_ops(ct + 1);
      f32x4 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kh = okh[ct & 1][s], kl = okl[ct & 1][s];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[rt][s], kh, acc[rt], 0, 0, 0);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[rt][s], kl, acc[rt], 0, 0, 0);
          if (kSplitQ) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[rt][s], kh, acc[rt], 0, 0, 0);
        }
      }
      const int jb = jc + l16;
      if constexpr (GS > 0) {
        // row tile rt: query 16 rt / H, heads 16 rt % H + 4 g16 + i, group (16 rt % H + 4 g16) / GS
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) p = fmaf(wv[rt][i], fmaxf(acc[rt][i], 0.f), p);
          if constexpr (GS == 8) p = row_pair_sum(p);     // lane groups 2m, 2m + 1 hold the pair's sum
          const int k = (16 * rt) / H;
          const int gi = ((16 * rt) % H + 4 * g16) / GS;
          const int qw = qa + wid * QW + k;
          if ((GS == 4 || (g16 & 1) == 0) && qw < qe && jb < ce) {
            const bool vis = jb >= vbk[k] && jb < vbk[k] + vnk[k];
            if (vis || write_invisible)
              otile[gi * gstride + static_cast<int64_t>(qw - qa) * ostride + (jb - j0)] = vis ? scale * p : -INFINITY;
          }
        }
        continue;
      }
      // weighted ReLU summed over each query's heads
      float part[QW];
#pragma unroll
      for (int k = 0; k < QW; ++k) part[k] = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = (16 * rt + 4 * g16 + i) / H;      // compile-time except for g16
#pragma unroll
          for (int kk = 0; kk < QW; ++kk)
            if (kk == k) part[kk] = fmaf(wv[rt][i], fmaxf(acc[rt][i], 0.f), part[kk]);
        }
      // lanes l, l^16, l^32, l^48 hold the same block: combine the head groups
#pragma unroll
      for (int k = 0; k < QW; ++k) {
        if (H >= 16) part[k] = row4_sum(part[k]);
        else if (H == 8) part[k] = row_pair_sum(part[k]);
      }
      if constexpr (H >= 16) {
        // every lane holds the sums of all QW (<= 4) queries: lane group g16
        // writes query g16, one store for the whole tile
        float v = part[0];
#pragma unroll
        for (int k = 1; k < QW; ++k) v = g16 == k ? part[k] : v;
        const bool vis = jb >= my_vb && jb < my_vb + my_vn;
        if (my_q && jb < ce && (vis || write_invisible))
          otile[my_off + (jb - j0)] = vis ? scale * v : -INFINITY;
      } else {
#pragma unroll
        for (int k = 0; k < QW; ++k) {
          // the lane group that owns query k's sum writes it
          const bool writer = H == 8 ? (g16 == 2 * (k % 2)) : (g16 == k % 4);
          const int qw = qa + wid * QW + k;
          if (writer && qw < qe && jb < ce) {
            const bool vis = jb >= vbk[k] && jb < vbk[k] + vnk[k];
            if (vis || write_invisible)
              otile[static_cast<int64_t>(qw - qa) * ostride + (jb - j0)] = vis ? scale * part[k] : -INFINITY;
          }
        }
      }
    }
    if constexpr (!kPre) {
      if (it + 1 < nch) lstore(buf ^ 1);
      __syncthreads();
    }
  }
}

// pre-split of the compressed keys for the streaming score path: per block a
// row of bf16 high halves, then a row of low halves
template <int D>
__global__ void __launch_bounds__(256)
split_keys_kernel(const float* __restrict__ kc, uint16_t* __restrict__ kcs, int64_t n_groups) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= n_groups) return;
  const int64_t blk = g / (D / 8);
  const int c8 = static_cast<int>(g % (D / 8));
  const float4 a = *reinterpret_cast<const float4*>(kc + blk * D + 8 * c8);
  const float4 b = *reinterpret_cast<const float4*>(kc + blk * D + 8 * c8 + 4);
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  bf16x8 hi, lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t h, l;
    split_bf16(f[e], h, l);
    hi[e] = static_cast<short>(h);
    lo[e] = static_cast<short>(l);
  }
  *reinterpret_cast<bf16x8*>(kcs + (blk * 2) * D + 8 * c8) = hi;
  *reinterpret_cast<bf16x8*>(kcs + (blk * 2 + 1) * D + 8 * c8) = lo;
}

template <typename QT, int D, int GS = 0>
static int launch_score_d(const Layout& L, const QT* q, int H, const float* w, const float* kc, const uint16_t* kcs,
                          const int32_t* cu_blocks, int c, float scale, int q0, int q1, int j0, int j1, float* out,
                          int64_t ostride, int write_invisible, int skip_nb, int n_grp, hipStream_t stream,
                          int64_t gstride = 0, const QPrep& prep = QPrep{}) {
  // one segment per row: measured on MI355X with bf16 queries, splitting rows
  // into segments of 512..1024 blocks was slower at S = 8192 and S = 131072
  // (each segment repeats the q-row loads and the pipeline fill), and the
  // latest-first order covers the causal imbalance; a third resident
  // workgroup (three key buffers) was slower too
  const int span = j1 - j0;
  int seg = std::max(1, span);
  seg = (seg + kScoreChunk - 1) / kScoreChunk * kScoreChunk;
  const int n_seg = (span + seg - 1) / seg;
  // queries per workgroup: 4 waves x 16 RT / H
  auto grid_for = [&](int rt, int h) {
    const int qg = 4 * (16 * rt / h);
    return dim3(static_cast<unsigned>(((q1 - q0 + qg - 1) / qg) * n_seg), static_cast<unsigned>(L.B));
  };
#define IRB_SCORE_CASE(HH)                                                                                   \
  case HH:                                                                                                   \
    if (kcs)                                                                                                 \
      hipLaunchKernelGGL((score_kernel<QT, D, HH, true, GS>), grid_for(score_rt<QT, D, HH, true>(), HH),    \
                         dim3(256), 0, stream, L, q, w, kc, kcs, cu_blocks, c, scale, q0, q1, j0, j1, out,    \
                         ostride, seg, n_seg, write_invisible, skip_nb, n_grp, gstride, prep);                \
    else                                                                                                     \
      hipLaunchKernelGGL((score_kernel<QT, D, HH, false, GS>), grid_for(score_rt<QT, D, HH, false>(), HH),  \
                         dim3(256), 0, stream, L, q, w, kc, kcs, cu_blocks, c, scale, q0, q1, j0, j1, out,    \
                         ostride, seg, n_seg, write_invisible, skip_nb, n_grp, gstride, prep);                \
    return 0;
  if constexpr (GS > 0) {
    switch (H) {
      IRB_SCORE_CASE(16)
      IRB_SCORE_CASE(32)
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  } else {
    switch (H) {
      IRB_SCORE_CASE(4)
      IRB_SCORE_CASE(8)
      IRB_SCORE_CASE(16)
      IRB_SCORE_CASE(32)
      IRB_SCORE_CASE(48)
      IRB_SCORE_CASE(64)
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
#undef IRB_SCORE_CASE
}

template <typename QT>
static int launch_score_t(const Layout& L, const QT* q, int H, int D, const float* w, const float* kc,
                          const uint16_t* kcs, const int32_t* cu_blocks, int c, float scale, int q0, int q1, int j0,
                          int j1, float* out, int64_t ostride, int write_invisible, int skip_nb, int n_grp,
                          hipStream_t stream, const QPrep& prep) {
  switch (D) {
    case 32: return launch_score_d<QT, 32>(L, q, H, w, kc, kcs, cu_blocks, c, scale, q0, q1, j0, j1, out, ostride, write_invisible, skip_nb, n_grp, stream, 0, prep);
    case 64: return launch_score_d<QT, 64>(L, q, H, w, kc, kcs, cu_blocks, c, scale, q0, q1, j0, j1, out, ostride, write_invisible, skip_nb, n_grp, stream, 0, prep);
    case 128: return launch_score_d<QT, 128>(L, q, H, w, kc, kcs, cu_blocks, c, scale, q0, q1, j0, j1, out, ostride, write_invisible, skip_nb, n_grp, stream, 0, prep);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int launch_split_keys(const float* kc, uint16_t* kcs, int64_t n_blocks, int D, hipStream_t stream) {
  const int64_t groups = n_blocks * (D / 8);
  const unsigned grid = static_cast<unsigned>((groups + 255) / 256);
  if (groups == 0) return 0;
  switch (D) {
    case 32: hipLaunchKernelGGL(split_keys_kernel<32>, dim3(grid), dim3(256), 0, stream, kc, kcs, groups); return 0;
    case 64: hipLaunchKernelGGL(split_keys_kernel<64>, dim3(grid), dim3(256), 0, stream, kc, kcs, groups); return 0;
    case 128: hipLaunchKernelGGL(split_keys_kernel<128>, dim3(grid), dim3(256), 0, stream, kc, kcs, groups); return 0;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int launch_score_tile(const Layout& L, const void* q, int dtype, int H, int D, const float* w,
                      const float* kc, const uint16_t* kc_split, const int32_t* cu_blocks, int c, float scale,
                      int q0, int q1, int j0, int j1, float* out, int64_t out_stride, int write_invisible,
                      int skip_nb, int n_grp, hipStream_t stream, const QPrep& prep) {
  if (prep.gamma && !score_prep_ok(D, prep.R)) return static_cast<int>(hipErrorInvalidValue);
  if (dtype == IRB_BF16)
    return launch_score_t(L, static_cast<const uint16_t*>(q), H, D, w, kc, kc_split, cu_blocks, c, scale, q0, q1, j0,
                          j1, out, out_stride, write_invisible, skip_nb, n_grp, stream, prep);
  return launch_score_t(L, static_cast<const float*>(q), H, D, w, kc, kc_split, cu_blocks, c, scale, q0, q1, j0, j1,
                        out, out_stride, write_invisible, skip_nb, n_grp, stream, prep);
}

bool score_grouped_ok(int dtype, int groups, int H_group, int D) {
  return dtype == IRB_BF16 && (H_group == 4 || H_group == 8) && groups > 1 &&
         (groups * H_group == 16 || groups * H_group == 32) && (D == 64 || D == 128);
}

int launch_score_grouped(const Layout& L, const void* q, int dtype, int groups, int H_group, int D, const float* w,
                         const float* kc, const uint16_t* kc_split, const int32_t* cu_blocks, int c, float scale,
                         int q0, int q1, int j0, int j1, float* out, int64_t out_stride, int64_t group_stride,
                         int write_invisible, int skip_nb, hipStream_t stream) {
  if (!score_grouped_ok(dtype, groups, H_group, D)) return static_cast<int>(hipErrorInvalidValue);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const int H = groups * H_group;
#define IRB_SCORE_GROUPED(DD, GG)                                                                           \
  return launch_score_d<uint16_t, DD, GG>(L, qb, H, w, kc, kc_split, cu_blocks, c, scale, q0, q1, j0, j1, out, \
                                          out_stride, write_invisible, skip_nb, 1, stream, group_stride);
  if (D == 64) {
    if (H_group == 4) { IRB_SCORE_GROUPED(64, 4) }
    IRB_SCORE_GROUPED(64, 8)
  }
  if (H_group == 4) { IRB_SCORE_GROUPED(128, 4) }
  IRB_SCORE_GROUPED(128, 8)
#undef IRB_SCORE_GROUPED
}

}  // namespace irb
