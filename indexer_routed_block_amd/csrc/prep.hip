// Index-query preparation: per (token, head) row, RMSNorm over the head
// dimension, then RoPE with the rotary row of the row's own token, composed in
// FP32 and rounded once to the activation dtype.
//
// QSA page (nemo_automodel...qwen3_8_flash_next.qsa): the indexer's
// q_layernorm and apply_qsa_rope (cat(cos, sin) rows; dimension i < D_rope/2
// pairs with i + D_rope/2; dimensions from D_rope on pass through);
// select_qsa_token_ids consumes the result as its normalised, rotated index
// queries.
//
// Each lane holds EPL consecutive dimensions of one row (16-byte loads and
// stores).  The D / EPL lanes of a row reduce the sum of squares with xor
// shuffles, and the rotation partner of a dimension is read from the wave's
// LDS copy of its normalised rows.  Rows are independent and each is read
// completely before it is written, so the output may alias the input.
#include "irb_internal.hpp"

namespace irb {

constexpr int kPrepWaves = 4;

template <typename T>
IRB_DEV void load16(const T* p, float* x);
template <>
IRB_DEV void load16<uint16_t>(const uint16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
IRB_DEV void load16<float>(const float* p, float* x) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

template <typename T>
IRB_DEV void store16(T* p, const float* y);
template <>
IRB_DEV void store16<uint16_t>(uint16_t* p, const float* y) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(y[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(y[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
IRB_DEV void store16<float>(float* p, const float* y) {
  *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
}

// A wavefront takes kPrepGroups groups of RPW rows; the loads of all its rows
// are issued before any is used, so each wave keeps several 16-byte row
// loads (and their rotary rows) in flight.
constexpr int kPrepGroups = 4;

template <typename T, int D>
__global__ void __launch_bounds__(kPrepWaves * 64)
prep_queries_kernel(const T* q, int64_t n_rows, int H, const float* __restrict__ gamma, float eps,
                    const float* __restrict__ rope, int R, int vec_tab, int xor_partner, T* out) {
  constexpr int VE = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte access
  constexpr int EPL = VE > D / 64 ? VE : D / 64;          // elements per lane
  constexpr int NV = EPL / VE;                             // 16-byte accesses per lane
  constexpr int LPR = D / EPL;                             // lanes per row (power of two)
  constexpr int RPW = 64 / LPR;                            // rows per wave and group
  constexpr int U = kPrepGroups;
  static_assert(LPR * EPL == D && RPW * LPR == 64, "row tiling");
  __shared__ float stage[kPrepWaves][64 * EPL];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kPrepWaves + wid) * (U * RPW) + sub;
  const bool small = n_rows < (int64_t{1} << 31);
  const int half = R / 2;
  float x[U][EPL], cs[U][EPL], sn[U][EPL], gm[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) gm[e] = gamma[li * EPL + e];
  // every row of this wave belongs to one token when H is a multiple of the
  // wave's U * RPW rows: the rotary factors are then loaded once
  const bool one_tok = H % (U * RPW) == 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = row0 + u * RPW;
    const int64_t rr = row < n_rows ? row : 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) load16<T>(q + rr * D + li * EPL + v * VE, x[u] + v * VE);
    if (u > 0 && one_tok) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        cs[u][e] = cs[0][e];
        sn[u][e] = sn[0][e];
      }
      continue;
    }
    // rotary factors: dimension d < R uses table entry j = d mod (R / 2),
    // rotated as x_d cos_j - x_{d + R/2} sin_j (first half) or
    // x_d cos_j + x_{d - R/2} sin_j (second half)
    const int64_t tok = small ? static_cast<int64_t>(static_cast<int>(rr) / H) : rr / H;
    const float* fr = R > 0 ? rope + tok * R : gamma;   // never read when R == 0; a valid address regardless
    if (vec_tab) {
      // D_rope / 2 a multiple of EPL (16-byte aligned rows): the lane's table
      // entries are EPL consecutive cos and EPL consecutive sin values
      const int d0 = li * EPL;
      const bool rot = d0 < R;
      const int j0 = d0 < half ? d0 : d0 - half;
      const float sg = d0 < half ? -1.f : 1.f;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 c4 = rot ? *reinterpret_cast<const float4*>(fr + j0 + e) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 s4 = rot ? *reinterpret_cast<const float4*>(fr + half + j0 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
        cs[u][e] = c4.x; cs[u][e + 1] = c4.y; cs[u][e + 2] = c4.z; cs[u][e + 3] = c4.w;
        sn[u][e] = sg * s4.x; sn[u][e + 1] = sg * s4.y; sn[u][e + 2] = sg * s4.z; sn[u][e + 3] = sg * s4.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = li * EPL + e;
        const bool rot = d < R;
        const int j = d < half ? d : d - half;
        cs[u][e] = rot ? fr[j] : 1.f;
        sn[u][e] = rot ? (d < half ? -fr[half + j] : fr[half + j]) : 0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t row = row0 + u * RPW;
    // the sum of squares and the rotation are written as explicit fmas so
    // that the scoring kernel's fused preparation rounds identically
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss = fmaf(x[u][e], x[u][e], ss);
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[u][e] = x[u][e] * inv * gm[e];
    float y[EPL];
    if (xor_partner) {
      // D_rope = D and D_rope / 2 a power-of-two multiple of EPL: the partner
      // of dim d (d +- D/2) is element e of lane lane ^ xor_partner
#pragma unroll
      for (int e = 0; e < EPL; ++e) y[e] = fmaf(x[u][e], cs[u][e], __shfl_xor(x[u][e], xor_partner, 64) * sn[u][e]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) stage[wid][lane * EPL + e] = x[u][e];
      wave_lds_sync();
      const float* mine = &stage[wid][sub * D];   // this row's normalised values
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = li * EPL + e;
        const int pd = d < half ? d + half : (d < R ? d - half : d);   // rotation partner (itself past R)
        y[e] = fmaf(x[u][e], cs[u][e], mine[pd] * sn[u][e]);
      }
      wave_lds_sync();                            // the stage is rewritten by the next group
    }
    if (row < n_rows) {
#pragma unroll
      for (int v = 0; v < NV; ++v) store16<T>(out + row * D + li * EPL + v * VE, y + v * VE);
    }
  }
}

int launch_prep_queries(const void* q, int dtype, int64_t n_rows, int H, int D, const float* gamma, float eps,
                        const float* rope, int R, void* out, hipStream_t stream) {
  if (n_rows == 0) return 0;
  // 16-byte table reads need D_rope / 2 to be a multiple of the lane's element
  // count (8 for bf16; max(4, D / 64) for FP32) and 16-byte aligned rows
  const int epl = dtype == IRB_BF16 ? (D / 64 > 8 ? D / 64 : 8) : (D / 64 > 4 ? D / 64 : 4);
  const int vec_tab = (R > 0 && (R / 2) % epl == 0 && (reinterpret_cast<uintptr_t>(rope) & 15) == 0) ? 1 : 0;
  // full-width rotation with the half width a power-of-two number of lanes:
  // the partner is a lane exchange (lane ^ (R / 2 / epl)) instead of LDS
  const int hl = R > 0 ? (R / 2) / epl : 0;
  const int xor_partner = (vec_tab && R == D && hl > 0 && (hl & (hl - 1)) == 0) ? hl : 0;
#define IRB_PREP_CASE(T, DD)                                                                                \
  case DD: {                                                                                                \
    constexpr int VE = 16 / static_cast<int>(sizeof(T));                                                    \
    constexpr int EPL = VE > DD / 64 ? VE : DD / 64;                                                        \
    constexpr int RPW = 64 / (DD / EPL);                                                                    \
    const int64_t per_block = static_cast<int64_t>(kPrepWaves) * kPrepGroups * RPW;                         \
    hipLaunchKernelGGL((prep_queries_kernel<T, DD>), dim3(static_cast<unsigned>((n_rows + per_block - 1) / per_block)), \
                       dim3(kPrepWaves * 64), 0, stream, static_cast<const T*>(q), n_rows, H, gamma, eps, rope, R, \
                       vec_tab, xor_partner, static_cast<T*>(out));                                         \
    return 0;                                                                                               \
  }
  if (dtype == IRB_BF16) {
    switch (D) {
      IRB_PREP_CASE(uint16_t, 32)
      IRB_PREP_CASE(uint16_t, 64)
      IRB_PREP_CASE(uint16_t, 128)
      IRB_PREP_CASE(uint16_t, 256)
      IRB_PREP_CASE(uint16_t, 512)
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
  switch (D) {
    IRB_PREP_CASE(float, 32)
    IRB_PREP_CASE(float, 64)
    IRB_PREP_CASE(float, 128)
    IRB_PREP_CASE(float, 256)
    IRB_PREP_CASE(float, 512)
    default: return static_cast<int>(hipErrorInvalidValue);
  }
#undef IRB_PREP_CASE
}

}  // namespace irb
