// a2: weighted-ReLU block scores on MFMA.
//
// CSA page (nemo_automodel...step5.sparse), indexer_score_tile: one bounded
// FP32 tile of scores sum_h w[t,h] * relu(q[t,h] . k[j]) with signed FP32
// head weights; visibility and scale per the QSA page, select_qsa_token_ids.
//
// Tiling.  A workgroup (4 waves) owns 512/H queries x 64 blocks.  Rows of the
// MFMA A operand are (query, head) pairs, columns are blocks, K is the index
// dimension.  The FP32 compressed keys of the tile are split once into bf16
// high and low halves in LDS; each wave keeps the operands of its 32 blocks
// in registers and streams its queries' rows from global memory, issuing
// q*hi + q*lo (plus q_lo*hi for FP32 queries) per 16x16x32 step.  The
// accumulator layout puts 4 heads of one query in each lane, so the head
// reduction is 4 in-lane FMAs plus at most two cross-lane adds.
#include "irb_internal.hpp"

namespace irb {

constexpr int kScoreBN = 64;   // blocks per workgroup
constexpr int kScoreRows = 512; // (query, head) rows per workgroup

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

template <typename QT, int D>
__global__ void __launch_bounds__(256)
score_kernel(Layout L, const QT* __restrict__ q, int H, const float* __restrict__ w,
             const float* __restrict__ kc, const int32_t* __restrict__ cu_blocks, int c, float scale,
             int q0, int q1, int j0, int j1, float* __restrict__ out, int64_t ostride, int n_jt) {
  constexpr int KS = D / 32;
  constexpr int LDK = D + 8;                 // padded LDS row (bf16 elements)
  constexpr bool kSplitQ = sizeof(QT) == 4;
  __shared__ uint16_t khi[kScoreBN * LDK];
  __shared__ uint16_t klo[kScoreBN * LDK];
  __shared__ int s_any;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.y;
  const int BQ = kScoreRows / H;
  const int qt = blockIdx.x / n_jt, jt = blockIdx.x % n_jt;
  const int qa = q0 + qt * BQ, qe = min(q1, qa + BQ);
  const int jb = j0 + jt * kScoreBN, je = min(j1, jb + kScoreBN);
  const int nb_max = L.S / c;

  if (tid == 0) s_any = 0;
  __syncthreads();
  for (int t = qa + tid; t < qe; t += 256) {
    const Doc d = doc_of(L, b, t);
    if (d.valid) {
      const int base = block_base(L, cu_blocks, d);
      const int nb = (t - d.start + 1) / c;
      if (max(base, jb) < min(base + nb, je)) s_any = 1;
    }
  }
  __syncthreads();
  float* otile = out + (static_cast<int64_t>(b) * (q1 - q0) + (qa - q0)) * ostride + (jb - j0);
  const int ncol = je - jb;
  if (!s_any) {
    for (int i = tid; i < (qe - qa) * kScoreBN; i += 256) {
      const int r = i / kScoreBN, cc = i % kScoreBN;
      if (cc < ncol) otile[static_cast<int64_t>(r) * ostride + cc] = -INFINITY;
    }
    return;
  }

  // stage the tile's compressed keys as bf16 hi/lo
  const float* kcb = kc + (static_cast<int64_t>(b) * nb_max) * D;
  for (int i = tid; i < kScoreBN * D / 4; i += 256) {
    const int r = i / (D / 4), c4 = (i % (D / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jb + r < je) v = *reinterpret_cast<const float4*>(kcb + static_cast<int64_t>(jb + r) * D + c4);
    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t h, l;
      split_bf16(f[e], h, l);
      khi[r * LDK + c4 + e] = h;
      klo[r * LDK + c4 + e] = l;
    }
  }
  __syncthreads();

  const int rh = wid >> 1, ch = wid & 1;
  const int g = lane >> 4, l16 = lane & 15;
  bf16x8 kh[2][KS], kl[2][KS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = (2 * ch + ct) * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kh[ct][s] = *reinterpret_cast<const bf16x8*>(&khi[col * LDK + 32 * s + 8 * g]);
      kl[ct][s] = *reinterpret_cast<const bf16x8*>(&klo[col * LDK + 32 * s + 8 * g]);
    }
  }

  // units: one query when H >= 16 (H/16 row tiles), else one row tile of 16/H queries
  const bool wide = H >= 16;
  const int tpu = wide ? H / 16 : 1;
  const int qpu = wide ? 1 : 16 / H;
  const int gpq = wide ? 4 : H / 4;          // lane groups per query inside a tile
  const int n_units = (qe - qa + qpu - 1) / qpu;
  const int64_t qrow = static_cast<int64_t>(H) * D;   // q elements per token

  for (int u = rh; u < n_units; u += 2) {
    float part[2] = {0.f, 0.f};
    for (int tq = 0; tq < tpu; ++tq) {
      // this lane's A row
      const int qi = qa + u * qpu + (wide ? 0 : l16 / H);
      const int hd = wide ? 16 * tq + l16 : l16 % H;
      bf16x8 qh[KS], ql[KS];
      const bool qok = qi < qe;
      const QT* qp = q + (static_cast<int64_t>(b) * L.S + (qok ? qi : qa)) * qrow + static_cast<int64_t>(hd) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        load_q_operand<QT>(qp + 32 * s, qh[s], ql[s]);
        if (!qok) {
#pragma unroll
          for (int e = 0; e < 8; ++e) { qh[s][e] = 0; if (kSplitQ) ql[s][e] = 0; }
        }
      }
      f32x4 acc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[s], kh[ct][s], acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[s], kl[ct][s], acc[ct], 0, 0, 0);
          if (kSplitQ) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[s], kh[ct][s], acc[ct], 0, 0, 0);
        }
      }
      // weighted relu over this lane's 4 rows (rows 4g..4g+3 of the tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const int qr = qa + u * qpu + (wide ? 0 : r / H);
        const int hr = wide ? 16 * tq + r : r % H;
        const float wv = (qr < qe) ? w[(static_cast<int64_t>(b) * L.S + qr) * H + hr] : 0.f;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) part[ct] += wv * fmaxf(acc[ct][i], 0.f);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (gpq >= 4) part[ct] = row4_sum(part[ct]);
      else if (gpq == 2) part[ct] = row_pair_sum(part[ct]);
    }
    if ((g % gpq) == 0) {
      const int qw = qa + u * qpu + g / gpq;
      if (qw < qe) {
        const Doc d = doc_of(L, b, qw);
        const int base = d.valid ? block_base(L, cu_blocks, d) : 0;
        const int nb = d.valid ? (qw - d.start + 1) / c : 0;
        float* orow = otile + static_cast<int64_t>(qw - qa) * ostride;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int cc = (2 * ch + ct) * 16 + l16;
          const int j = jb + cc;
          if (cc < ncol) orow[cc] = (j >= base && j < base + nb) ? scale * part[ct] : -INFINITY;
        }
      }
    }
  }
}

template <typename QT>
static int launch_score_t(const Layout& L, const QT* q, int H, int D, const float* w, const float* kc,
                          const int32_t* cu_blocks, int c, float scale, int q0, int q1, int j0, int j1,
                          float* out, int64_t ostride, hipStream_t stream) {
  const int BQ = kScoreRows / H;
  const int n_qt = (q1 - q0 + BQ - 1) / BQ;
  const int n_jt = (j1 - j0 + kScoreBN - 1) / kScoreBN;
  const dim3 grid(static_cast<unsigned>(n_qt * n_jt), static_cast<unsigned>(L.B));
  const dim3 block(256);
#define IRB_SCORE_CASE(DD)                                                                              \
  case DD:                                                                                              \
    hipLaunchKernelGGL((score_kernel<QT, DD>), grid, block, 0, stream, L, q, H, w, kc, cu_blocks, c, scale, \
                       q0, q1, j0, j1, out, ostride, n_jt);                                            \
    break;
  switch (D) {
    IRB_SCORE_CASE(32)
    IRB_SCORE_CASE(64)
    IRB_SCORE_CASE(128)
    default: return static_cast<int>(hipErrorInvalidValue);
  }
#undef IRB_SCORE_CASE
  return 0;
}

int launch_score_tile(const Layout& L, const void* q, int dtype, int H, int D, const float* w,
                      const float* kc, const int32_t* cu_blocks, int c, float scale, int q0, int q1,
                      int j0, int j1, float* out, int64_t out_stride, hipStream_t stream) {
  if (dtype == IRB_BF16)
    return launch_score_t(L, static_cast<const uint16_t*>(q), H, D, w, kc, cu_blocks, c, scale, q0, q1, j0, j1,
                          out, out_stride, stream);
  return launch_score_t(L, static_cast<const float*>(q), H, D, w, kc, cu_blocks, c, scale, q0, q1, j0, j1, out,
                        out_stride, stream);
}

}  // namespace irb
