// a6: sparse GQA attention forward over routed (gathered) keys.
//
// QSA page (nemo_automodel...qwen3_8_flash_next.qsa), gathered_qsa_gqa_attention
// and qsa_gqa_attention: each query attends to the keys/values at its route
// IDs only, grouped heads share a KV head, no K/V head expansion; latent page
// (common.cudnn_sparse_attention), cudnn_sparse_attention: one shared latent
// KV row per token, value = its first Dv channels.
//
// Work item = (batch, query, KV head).  The route is consumed in chunks of 32
// keys.  MFMA orientation (16x16x32 bf16, FP32 accumulate):
//   S^T[key, head] = K_chunk . Q^T      A = gathered K rows, B = resident Q
//   O^T[dim, head] += V_chunk^T . P^T   A = V^T read from LDS, B = P^T straight
//                                        from the S^T accumulators
// so softmax statistics live per lane (column = head) and no accumulator is
// ever moved between lanes except for the max/sum butterflies.
// G <= 16: one wavefront per item, K rows gathered straight into registers,
//          V rows staged in a per-wave LDS slab for the transposed read.
// G > 16:  one workgroup per item, one wavefront per 16 heads; K and V chunks
//          staged once in LDS and shared (for latent KV a single slab).
// FP32 inputs are split into bf16 high/low parts (three MFMAs per product).
#include <cstdlib>

#include "irb_internal.hpp"

namespace irb {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;



IRB_DEV void ld8(const uint16_t* p, bf16x8& hi, bf16x8& lo) {
  hi = *reinterpret_cast<const bf16x8*>(p);
  (void)lo;
}
IRB_DEV void ld8(const float* p, bf16x8& hi, bf16x8& lo) {
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
IRB_DEV void zero8(bf16x8& x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0;
}
IRB_DEV void put(bf16x8& hi, bf16x8& lo, int e, uint16_t v) { hi[e] = static_cast<short>(v); (void)lo; }
IRB_DEV void put(bf16x8& hi, bf16x8& lo, int e, float v) {
  uint16_t h, l;
  split_bf16(v, h, l);
  hi[e] = static_cast<short>(h);
  lo[e] = static_cast<short>(l);
}
IRB_DEV void put_p(bf16x8& hi, bf16x8& lo, int e, float v, bool split) {
  if (split) {
    uint16_t h, l;
    split_bf16(v, h, l);
    hi[e] = static_cast<short>(h);
    lo[e] = static_cast<short>(l);
  } else {
    hi[e] = static_cast<short>(f32_to_bf16(v));
  }
}

template <bool kSplit>
IRB_DEV f32x4 mma(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  if (kSplit) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  }
  return acc;
}

IRB_DEV void store4(uint16_t* p, const float* v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
IRB_DEV void store4(float* p, const float* v) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }

template <typename T>
IRB_DEV int pad_elems() { return sizeof(T) == 2 ? 8 : 4; }

// copy one 16-byte vector of a gathered row into LDS (zeros for invalid rows)
IRB_DEV void copy16(void* dst, const void* src, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *reinterpret_cast<const uint4*>(src);
  *reinterpret_cast<uint4*>(dst) = v;
}

// kDelta: instead of o and lse, write Delta[b, h, t] = sum_d dO[t,h,d] * o[t,h,d]
// with o held in FP32 (the backward's row statistic, free of the rounding of
// the stored bf16 output).
// One (batch, query, KV head) item over its route.  kShared: called by every
// wave of the workgroup (wave = 16-head slice), K/V chunks staged in `smem`
// shared by all waves; otherwise called by one wave with `smem` its own slab.
template <typename T, int D, int DV, bool kShared, bool kDelta>
IRB_DEV void fwd_item(const AttnArgs& a, T* __restrict__ out, float* __restrict__ lse, int G, int latent,
                      const T* __restrict__ dout, float* __restrict__ delta, int b, int t, int kvh, int slice,
                      char* smem) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int KS = D / 32;
  constexpr int NDT = DV / 16;
  constexpr int PAD = sizeof(T) == 2 ? 8 : 4;
  constexpr int LDK = D + PAD;
  constexpr int LDV = DV + PAD;
  const int lane = threadIdx.x & 63;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int h0 = kvh * G + 16 * slice;
  const int nh = min(16, G - 16 * slice);
  const T* qbase = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t;
  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;

  bf16x8 qh[KS], ql[KS];
  {
    const bool ok = l16 < nh;
    const T* qp = qbase + static_cast<int64_t>(h0 + (ok ? l16 : 0)) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      ld8(qp + 32 * s, qh[s], ql[s]);
      if (!ok) { zero8(qh[s]); zero8(ql[s]); }
    }
  }
  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY, lsum = 0.f;
  const float sc2 = a.scale * kLog2e;

  T* kl = reinterpret_cast<T*>(smem);
  T* vl;
  int ldv;
  if (kShared) {
    vl = latent ? kl : kl + 32 * LDK;
    ldv = latent ? LDK : LDV;
  } else {
    vl = reinterpret_cast<T*>(smem);
    ldv = LDV;
  }

  for (int e0 = 0; e0 < n; e0 += 32) {
    // ---- stage the chunk's V rows (and K rows when shared) in LDS
    if (kShared) {
      __syncthreads();
      constexpr int KV16 = D * static_cast<int>(sizeof(T)) / 16;
      for (int i = threadIdx.x; i < 32 * KV16; i += blockDim.x) {
        const int kk = i / KV16, c16 = i % KV16;
        const int e = e0 + kk;
        const int id = e < n ? route[e] : -1;
        const bool ok = id >= 0 && id < a.S_k;
        copy16(reinterpret_cast<char*>(kl + kk * LDK) + 16 * c16,
               reinterpret_cast<const char*>(kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t) + 16 * c16, ok);
      }
      if (!latent) {
        constexpr int V16 = DV * static_cast<int>(sizeof(T)) / 16;
        for (int i = threadIdx.x; i < 32 * V16; i += blockDim.x) {
          const int kk = i / V16, c16 = i % V16;
          const int e = e0 + kk;
          const int id = e < n ? route[e] : -1;
          const bool ok = id >= 0 && id < a.S_k;
          copy16(reinterpret_cast<char*>(vl + kk * LDV) + 16 * c16,
                 reinterpret_cast<const char*>(vbase + static_cast<int64_t>(ok ? id : 0) * a.sv_t) + 16 * c16, ok);
        }
      }
      __syncthreads();
    } else {
      constexpr int V16 = DV * static_cast<int>(sizeof(T)) / 16;
      const int kk = lane >> 1, hf = lane & 1;
      const int e = e0 + kk;
      const int id = e < n ? route[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      const char* src = reinterpret_cast<const char*>(vbase + static_cast<int64_t>(ok ? id : 0) * a.sv_t);
      char* dst = reinterpret_cast<char*>(vl + kk * LDV);
      for (int c16 = hf; c16 < V16; c16 += 2) copy16(dst + 16 * c16, src + 16 * c16, ok);
      wave_lds_sync();
    }

    // ---- S^T = K Q^T for two tiles of 16 keys
    f32x4 st[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      st[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (kShared) {
        const T* kr = kl + (16 * ti + l16) * LDK + 8 * g16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          bf16x8 kh, klo;
          ld8(kr + 32 * s, kh, klo);
          st[ti] = mma<kSplit>(kh, klo, qh[s], ql[s], st[ti]);
        }
      } else {
        const int e = e0 + 16 * ti + l16;
        const int id = e < n ? route[e] : -1;
        const bool ok = id >= 0 && id < a.S_k;
        const T* kr = kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t + 8 * g16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          bf16x8 kh, klo;
          ld8(kr + 32 * s, kh, klo);
          if (!ok) { zero8(kh); zero8(klo); }
          st[ti] = mma<kSplit>(kh, klo, qh[s], ql[s], st[ti]);
        }
      }
    }

    // ---- online softmax over this chunk; column = head l16
    float x[2][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * ti + 4 * g16 + i;
        x[ti][i] = (e < n) ? st[ti][i] * sc2 : -INFINITY;
        cmax = fmaxf(cmax, x[ti][i]);
      }
    cmax = row4_max(cmax);
    const float mnew = fmaxf(m2, cmax);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;   // nothing visible yet: every p is 0
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) { p[ti][i] = fast_exp2(x[ti][i] - mref); ps += p[ti][i]; }
    const float alpha = fast_exp2(m2 - mref);
    m2 = mnew;
    lsum = lsum * alpha + ps;
    if (__ballot(alpha != 1.f)) {           // rescale only when some head's max moved
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;
    }

    // P^T operand: k positions 8*g16 + j <-> keys {4g..4g+3} of tile 0, then of tile 1
    bf16x8 ph, pl;
    if (kSplit) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        put_p(ph, pl, j, p[0][j], true);
        put_p(ph, pl, 4 + j, p[1][j], true);
      }
    } else {
      const float pf[8] = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
      ph = pack_bf16x8(pf);
    }
    // ---- O^T += V^T P^T; A operand read transposed from LDS
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      bf16x8 vh, vlo;
      const T* vc = vl + dt * 16 + l16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = (j < 4) ? 4 * g16 + j : 16 + 4 * g16 + (j - 4);
        put(vh, vlo, j, vc[kk * ldv]);
      }
      oacc[dt] = mma<kSplit>(vh, vlo, ph, pl, oacc[dt]);
    }
    if (!kShared) {
      wave_lds_sync();
    }
  }

  float ltot = row4_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (kDelta) {
    float part = 0.f;
    if (l16 < nh) {
      const T* dp = dout + (row * a.Hq + h0 + l16) * DV + 4 * g16;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += oacc[dt][i] * inv * load_as_f32(dp + dt * 16 + i);
    }
    part = row4_sum(part);
    if (l16 < nh && g16 == 0) delta[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = part;
    return;
  }
  if (l16 < nh) {
    T* op = out + (row * a.Hq + h0 + l16) * DV + 4 * g16;
    float* o32 = a.o32 ? a.o32 + (row * a.Hq + h0 + l16) * DV + 4 * g16 : nullptr;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float v[4] = {oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv};
      store4(op + dt * 16, v);
      if (o32) store4(o32 + dt * 16, v);
    }
    if (g16 == 0)
      lse[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = ltot > 0.f ? (m2 + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// bf16, one wavefront per (batch, query, KV head) with G <= 16 heads as the
// MFMA columns.  The next chunk's K rows (A-layout registers) and V rows
// (registers, then the wave's LDS slab) are loaded while the current chunk is
// computed; V^T operands come from the slab by LDS transpose reads.
template <int D, int DV, bool kDelta>
IRB_DEV void fwd_item_gather(const AttnArgs& a, uint16_t* __restrict__ out, float* __restrict__ lse, int G,
                             const uint16_t* __restrict__ dout, float* __restrict__ delta, int b, int t, int kvh,
                             char* smem) {
  using T = uint16_t;
  constexpr int KS = D / 32;
  constexpr int NDT = DV / 16;
  constexpr int LDV = DV + 8;
  constexpr int VU = DV / 16;                 // 16-byte V chunks per lane (two lanes per row)
  const int lane = threadIdx.x & 63;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int h0 = kvh * G;
  const int nh = min(16, G);
  const T* qbase = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t;
  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;

  bf16x8 qh[KS];
  {
    const bool ok = l16 < nh;
    const T* qp = qbase + static_cast<int64_t>(h0 + (ok ? l16 : 0)) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qh[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
      if (!ok) zero8(qh[s]);
    }
  }
  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY, lsum = 0.f;
  const float sc2 = a.scale * kLog2e;
  T* vl = reinterpret_cast<T*>(smem);
  const int vkk = lane >> 1, vhf = lane & 1;         // V staging: row, half
  const int vk0 = 4 * g16 + (l16 >> 2);              // V^T transpose reads: first key row

  struct Pre { bf16x8 k[2][KS]; uint4 v[VU]; };
  auto load = [&](int e0, Pre& r) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int e = e0 + 16 * ti + l16;
      const int id = e < n ? route[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      const T* kr = kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t + 8 * g16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        r.k[ti][s] = *reinterpret_cast<const bf16x8*>(kr + 32 * s);
        if (!ok) zero8(r.k[ti][s]);
      }
    }
    const int e = e0 + vkk;
    const int id = e < n ? route[e] : -1;
    const bool ok = id >= 0 && id < a.S_k;
    const T* vr = vbase + static_cast<int64_t>(ok ? id : 0) * a.sv_t;
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      r.v[u] = ok ? *reinterpret_cast<const uint4*>(vr + 8 * (vhf + 2 * u)) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // one register set: the chunk's V rows go to the slab and its K rows into
  // the S MFMAs, then the set is refilled with the next chunk, whose loads
  // overlap this chunk's softmax and PV work
  auto step = [&](int e0, Pre& pf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VU; ++u) *reinterpret_cast<uint4*>(vl + vkk * LDV + 8 * (vhf + 2 * u)) = pf.v[u];
    // ---- S^T = K Q^T for two tiles of 16 keys
    f32x4 st[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      st[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) st[ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf.k[ti][s], qh[s], st[ti], 0, 0, 0);
    }
    wave_lds_sync();
    if (e0 + 32 < n) load(e0 + 32, pf);
    // ---- online softmax over this chunk; column = head l16
    float x[2][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * ti + 4 * g16 + i;
        x[ti][i] = (e < n) ? st[ti][i] * sc2 : -INFINITY;
        cmax = fmaxf(cmax, x[ti][i]);
      }
    cmax = row4_max(cmax);
    const float mnew = fmaxf(m2, cmax);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) { p[4 * ti + i] = fast_exp2(x[ti][i] - mref); ps += p[4 * ti + i]; }
    const float alpha = fast_exp2(m2 - mref);
    m2 = mnew;
    lsum = lsum * alpha + ps;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;
    }
    const bf16x8 pop = pack_bf16x8(p);
    // ---- O^T += V^T P^T; k-slot j is key 4 g16 + j (j < 4) or 16 + 4 g16 + (j - 4)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const T* w = vl + vk0 * LDV + 16 * dt + 4 * (l16 & 3);
      const v4s v0 = lds_read_tr(w), v1 = lds_read_tr(w + 16 * LDV);
      const bf16x8 vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, oacc[dt], 0, 0, 0);
    }
    wave_lds_sync();   // the slab is rewritten by the next chunk
  };
  if (n > 0) {
    Pre pf;
    load(0, pf);
    for (int e0 = 0; e0 < n; e0 += 32) step(e0, pf);
  }

  float ltot = row4_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (kDelta) {
    float part = 0.f;
    if (l16 < nh) {
      const T* dp = dout + (row * a.Hq + h0 + l16) * DV + 4 * g16;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += oacc[dt][i] * inv * bf16_to_f32(dp[dt * 16 + i]);
    }
    part = row4_sum(part);
    if (l16 < nh && g16 == 0) delta[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = part;
    return;
  }
  if (l16 < nh) {
    T* op = out + (row * a.Hq + h0 + l16) * DV + 4 * g16;
    float* o32 = a.o32 ? a.o32 + (row * a.Hq + h0 + l16) * DV + 4 * g16 : nullptr;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float v[4] = {oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv};
      store4(op + dt * 16, v);
      if (o32) store4(o32 + dt * 16, v);
    }
    if (g16 == 0)
      lse[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = ltot > 0.f ? (m2 + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Query-tile kernel for dense-ish routes (G <= 16, bf16).
//
// Work item = (batch, tile of BQ = 128/G consecutive queries, KV head): 128
// (query, head) columns, 32 per wave.  The key tiles (32 keys) any query of
// the tile routes to are streamed through double-buffered LDS as contiguous
// rows, K as [key][dim] and V transposed to [dim][key] on the way in, both
// shared by all 128 columns:
//   S^T[key, col] = K_tile . Q^T       A = K from LDS, B = resident Q
//   O^T[dim, col] += V_tile^T . P^T    A = V^T from LDS (two 8-byte reads),
//                                      B = P^T straight from S^T
// Route membership enters as one 32-bit mask word per (query, key tile),
// built in LDS per segment of 8192 keys from each query's sorted route (one
// binary search per query and segment, then independent coalesced reads with
// equal words OR-combined across lanes before one atomic per word).  The tile's cost is (key tiles touched) x
// 128 columns of MFMA work, so a tile is taken here only when its route
// entries fill at least thr/1000 of (valid queries x key span); the gather
// kernel handles the other tiles (both kernels evaluate the same integer test).

template <typename T, int D, int DV, bool kShared, bool kDelta>
__global__ void __launch_bounds__(256, (kShared || D > 128 || sizeof(T) == 4) ? 1 : 3)
attn_fwd_kernel(AttnArgs a, T* __restrict__ out, float* __restrict__ lse, int G, int n_items, int latent,
                const T* __restrict__ dout, float* __restrict__ delta, int tile_bq, int thr_milli, int head_major) {
  constexpr int PAD = sizeof(T) == 2 ? 8 : 4;
  extern __shared__ __align__(16) char smem[];
  const int wid = threadIdx.x >> 6;
  int item, slice;
  char* slab = smem;
  if (kShared) {
    item = blockIdx.x;
    slice = wid;
  } else {
    item = blockIdx.x * 4 + wid;
    slice = 0;
    if (item >= n_items) return;
    slab = smem + static_cast<size_t>(wid) * 32 * (DV + PAD) * sizeof(T);
  }
  const QItem qi = decode_qitem(item, a.B, a.S_q, a.Hkv, kShared ? 0 : head_major);
  const int kvh = qi.kvh, t = qi.t, b = qi.b;
  if (!kShared && tile_bq > 0 && tile_stats_wave(a, b, kvh, (t / tile_bq) * tile_bq, tile_bq, thr_milli).dense) return;
  if constexpr (!kShared && sizeof(T) == 2 && D <= 128)
    fwd_item_gather<D, DV, kDelta>(a, out, lse, G, dout, delta, b, t, kvh, slab);
  else
    fwd_item<T, D, DV, kShared, kDelta>(a, out, lse, G, latent, dout, delta, b, t, kvh, slice, slab);
}

template <int D, int DV, int G, bool kDelta>
__global__ void __launch_bounds__(256, 2)
attn_fwd_tile_kernel(AttnArgs a, uint16_t* __restrict__ out, float* __restrict__ lse, const uint16_t* __restrict__ dout,
                     float* __restrict__ delta, int n_qt, int thr_milli, const uint32_t* __restrict__ qbits,
                     int qwords, int gather_rest) {
  using T = uint16_t;
  constexpr int BQ = 128 / G;
  constexpr int KS = D / 16;          // 16-dim k-steps of S^T = K Q^T
  constexpr int NDT = DV / 32;        // 32-dim row tiles of O^T
  constexpr int NG = KS;              // MFMA groups per step (one S and one O MFMA each)
  static_assert(D == DV && 2 * NDT == NG, "one S and one O MFMA per group");
  // K and V tiles are row-major (one key per row, no padding), filled by
  // direct global-to-LDS loads (lane i of a load writes 16-byte slot i).  The
  // 16-byte chunks of row r sit XOR-swizzled: chunk c of a K row at slot
  // c ^ (r mod NCK), of a V row at slot c ^ tr_swz(r), so the K operand
  // reads of 16 rows and the 32-lane V^T transpose reads (4 rows x 4 chunks;
  // the reads 8 and 16 rows further use the same pattern) hit distinct banks.
  // Three slots, each holding one tile's K and V.
  constexpr int NCK = D / 8, NCV = DV / 8;            // 16-byte chunks per row
  constexpr int KBYTES = 32 * D * 2, VBYTES = 32 * DV * 2;
  constexpr int BUF = KBYTES + VBYTES;
  constexpr int NIK = 32 * NCK / 256, NIV = 32 * NCV / 256;   // loads per wave per tile
  static_assert(NIK >= 1 && NIV >= 1, "tile loads");
  __shared__ __align__(16) char raw[3 * BUF];
  // key tiles per mask segment: halved where a full segment's mask rows
  // would leave LDS for only one workgroup per CU (G = 4 at D = 128: 32
  // query rows next to 48 KiB of K/V slots)
  constexpr int SEG = 3 * BUF + BQ * (kSegTiles + 1) * 4 > 78 * 1024 ? kSegTiles / 2 : kSegTiles;
  // one padding word per row: the softmax reads the words of a wave's four
  // queries at once, and rows a multiple of 256 words apart share a bank
  __shared__ uint32_t mask[BQ][SEG + 1];
  __shared__ int tiles[SEG];
  __shared__ int s_ntiles;
  __shared__ int cursor[BQ];
  __shared__ int s_lo[BQ], s_hi[BQ];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  // consecutive workgroups take the KV heads of one query tile (one head per
  // XCD when 8 is a multiple of Hkv, keeping that head's K/V in its L2), and
  // query tiles run last-first: causal tiles late in the sequence span the
  // most keys, so the heavy ones start early and the grid ends on light ones
  const int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  const int qt = n_qt - 1 - (bid / a.Hkv) % n_qt;
  const int b = bid / (a.Hkv * n_qt);
  const int qa = qt * BQ;
  const TileStats ts = tile_stats_wave(a, b, kvh, qa, BQ, thr_milli);
  if (!ts.dense) {
    // a sparse tile is the gather kernel's, or, when this launch takes every
    // tile (gather_rest), gathered here: wave w takes queries w, w + 4, ...
    // with its own slab of the (so far unused) K/V slots
    if (!gather_rest) return;
    char* slab = raw + wid * 32 * (DV + 8) * 2;
    static_assert(4 * 32 * (DV + 8) * 2 <= 3 * BUF, "gather slabs");
    for (int q = wid; q < BQ; q += 4)
      if (qa + q < a.S_q) fwd_item_gather<D, DV, kDelta>(a, out, lse, G, dout, delta, b, qa + q, kvh, slab);
    return;
  }

  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  // this lane's column: (query, head) pair 32 wid + l32; MFMA layout
  // (v_mfma_f32_32x32x16_bf16): A lane l = row l % 32, k 8 (l / 32) .. + 8;
  // B lane l = column l % 32, same k; accumulator element i of lane l =
  // row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
  const int col = 32 * wid + l32;
  const int colq = col / G, colh = col % G;
  bf16x8 qop[KS];
  {
    const int t = qa + colq;
    const bool ok = t < a.S_q;
    const T* qp = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(ok ? t : 0) * a.sq_t +
                  static_cast<int64_t>(kvh * G + colh) * a.sq_h + 8 * h32;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      qop[s2] = *reinterpret_cast<const bf16x8*>(qp + 16 * s2);
      if (!ok) zero8(qop[s2]);
    }
  }
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m2 = -INFINITY, lsum = 0.f;
  const float sc2 = a.scale * kLog2e;

  // tile loader: wave w issues NIK (K) or NIV (V) direct loads per tile;
  // lane i of load n fills slot (w NI + n) 64 + i.  The global address is the
  // tile's first row (wave-uniform, scalar registers) plus a per-lane 32-bit
  // byte offset fixed for the whole kernel; only a tile reaching past the
  // last key recomputes it with clamped rows.
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  uint32_t koff[NIK], voff[NIV];
#pragma unroll
  for (int n = 0; n < NIK; ++n) {
    const int slot = (wv * NIK + n) * 64 + lane;
    const int r = slot / NCK, sc = slot % NCK;
    koff[n] = static_cast<uint32_t>(r * a.sk_t + 8 * (sc ^ (r & (NCK - 1)))) * 2u;
  }
#pragma unroll
  for (int n = 0; n < NIV; ++n) {
    const int slot = (wv * NIV + n) * 64 + lane;
    const int r = slot / NCV, sc = slot % NCV;
    voff[n] = static_cast<uint32_t>(r * a.sv_t + 8 * (sc ^ tr_swz<NCV>(r))) * 2u;
  }
  const uint32_t lds0 = lds_addr(raw);
  // K rows of key tile kt into slot `buf` (kV = false) or its V rows (kV = true)
  auto issue = [&](int kt, auto bufc, auto vc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    constexpr bool kV = decltype(vc)::value;
    constexpr int NI = kV ? NIV : NIK, NC = kV ? NCV : NCK;
    kt = __builtin_amdgcn_readfirstlane(kt);
    const int key0 = kt * 32;
    const T* src = kV ? vbase + static_cast<int64_t>(key0) * a.sv_t : kbase + static_cast<int64_t>(key0) * a.sk_t;
    const int stride = kV ? a.sv_t : a.sk_t;
    const int lim = a.S_k - 1 - key0;
    const uint32_t ld = lds0 + buf * BUF + (kV ? KBYTES : 0) + wv * NI * 1024;
    if (lim >= 31) {
#pragma unroll
      for (int n = 0; n < NI; ++n) lds_dma16_s(src, kV ? voff[n] : koff[n], ld + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int slot = (wv * NI + n) * 64 + lane;
        const int r = slot / NC, sc = slot % NC;
        const int sw = kV ? (sc ^ tr_swz<NC>(r)) : (sc ^ (r & (NC - 1)));
        lds_dma16_s(src, static_cast<uint32_t>(min(r, lim) * stride + 8 * sw) * 2u, ld + n * 1024);
      }
    }
  };
  using KSide = std::integral_constant<bool, false>;
  using VSide = std::integral_constant<bool, true>;
  // per-lane LDS byte offsets inside a slot.  K operand of k-step s2: row
  // l32, chunk 2 s2 + h32.  V^T operand of dim tile dt: lanes of a 16-lane
  // row address keys r0 + (lane % 16) / 4 and dims 32 dt + 16 ((lane / 16) % 2)
  // + 4 (lane % 4), r0 = 4 h32 (+ 8 for the upper four k of a step, + 16
  // for the second step: whole rows, same swizzle, so immediate offsets)
  uint32_t kofs[KS], vofs[NDT];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) kofs[s2] = static_cast<uint32_t>(l32 * D + 8 * ((2 * s2 + h32) ^ (l32 & (NCK - 1)))) * 2u;
  {
    const int s16 = lane & 15, g2 = (lane >> 4) & 1;
    const int vr = 4 * h32 + (s16 >> 2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int vc = 4 * dt + 2 * g2 + ((s16 & 3) >> 1);
      vofs[dt] = static_cast<uint32_t>(vr * DV + 8 * (vc ^ tr_swz<NCV>(vr)) + 4 * (s16 & 1)) * 2u;
    }
  }
  // S^T of the key tile in the slot at byte offset kslot
  auto scores = [&](f32x16& st, uint32_t kslot) __attribute__((always_inline)) {
    const char* kb = raw + kslot;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kb + kofs[s2]), qop[s2], st, 0, 0, 0);
  };
  // V^T operand of dim tile dt, k-step t2 (keys 16 t2 + 4 h32 + {0..3, 8..11}),
  // from the V rows of the slot at byte offset vslot
  auto vread = [&](int dt, int t2, uint32_t vslot) __attribute__((always_inline)) {
    const char* vt = raw + vslot + KBYTES + vofs[dt] + t2 * 16 * DV * 2;
    const v4s v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vt));
    const v4s v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vt + 8 * DV * 2));
    return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  };
  // O^T += V^T P^T for the V rows in slot vslot (both k-steps of every dim tile)
  auto accumulate = [&](const bf16x8 (&pp)[2], uint32_t vslot) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(dt, t2, vslot), pp[t2], oacc[dt], 0, 0, 0);
  };

  // Software pipeline over the key tiles of a segment (n of them): step i
  // forms S^T of tile i + 1, the softmax of tile i and O^T += V^T P^T of
  // tile i - 1, three independent streams interleaved group by group (one S
  // MFMA, one O MFMA and a slice of the softmax arithmetic per group), so the
  // MFMAs of a wavefront run under its own VALU work.  Tile t's K rows sit in
  // slot t % 3 and its V rows in the V half of slot t % 3.  Step i first
  // waits for K(i + 1) and V(i - 1), then the barrier frees K slot i % 3
  // (read by S(i) in step i - 1) and V slot (i + 1) % 3 (read by step i - 1),
  // which receive K(i + 3) and V(i + 1).  Loads are issued in the order
  // K(0) K(1) K(2) V(0) | K(3) V(1) | K(4) V(2) | ..., so "everything but
  // the batch of step i - 1" is one vmcnt.
  f32x16 scur;
  bf16x8 pprev[2];
  // Values a step needs before its first MFMA, read from LDS one step ahead
  // (so that no step starts with a chain of LDS round trips): the key tiles
  // whose K (nk = tiles[i + 3]) and V (nv = tiles[i + 1]) rows step i
  // loads, and this lane's mask word of tile i (nmw).  Indices past the
  // list are clamped; their values go unused.
  int nk = 0, nv = 0;
  uint32_t nmw = 0u;
  auto step = [&](auto cc, auto pvc, int i, int ntiles, int seg0) __attribute__((always_inline)) {
    constexpr int C = decltype(cc)::value;      // i % 3
    constexpr bool kPV = decltype(pvc)::value;  // i > 0
    if (i + 2 < ntiles) __builtin_amdgcn_s_waitcnt(kDmaWait<NIK + NIV>());
    else __builtin_amdgcn_s_waitcnt(kDmaWait<NIV>());
    bare_barrier();
    const int tk = __builtin_amdgcn_readfirstlane(nk), tv = __builtin_amdgcn_readfirstlane(nv);
    if (i + 3 < ntiles) issue(seg0 + tk, std::integral_constant<int, C>{}, KSide{});
    if (i + 1 < ntiles) issue(seg0 + tv, std::integral_constant<int, (C + 1) % 3>{}, VSide{});
    const uint32_t mw = nmw >> (4 * h32);
    nk = tiles[min(i + 4, ntiles - 1)];
    nv = tiles[min(i + 2, ntiles - 1)];
    nmw = mask[colq][tv];
    constexpr uint32_t kslot = ((C + 1) % 3) * BUF, vslot = ((C + 2) % 3) * BUF;
    const char* kb = raw + kslot;
    // Masked online softmax of tile i in this lane's column, in eight pieces
    // spread over the MFMA groups: 0/1 mask select of elements 0-7 / 8-15
    // (an entry whose mask bit is clear becomes -inf by a bit select with the
    // sign-extended bit), 2 the in-lane max, 3 the max across the two lane
    // halves and the update of the reference max, 4-7 the exponentials.  The
    // reference max m2 only moves when a score exceeds it by more than kLazy
    // (log2 units), so weights stay <= 2^kLazy and the rescale of the
    // accumulators is rare; the result is exact after normalisation by lsum.
    // All branch-free, so the step is one scheduling region.
    constexpr float kLazy = 8.f;
    float xr[16], p[16];
    float cm = -INFINITY, mprev = 0.f, nm = 0.f;
    bool rescale = false;
    auto piece = [&](int pc) __attribute__((always_inline)) {
      if (pc < 2) {
#pragma unroll
        for (int i = 8 * pc; i < 8 * pc + 8; ++i) {
          const int bit = 8 * (i >> 2) + (i & 3);
          const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(mw << (31 - bit)) >> 31);
          xr[i] = __uint_as_float((__float_as_uint(scur[i]) & m) | (~m & 0xff800000u));
        }
      } else if (pc == 2) {
        const float x0 = max3_raw(xr[0], xr[1], xr[2]), x1 = max3_raw(xr[3], xr[4], xr[5]);
        const float x2 = max3_raw(xr[6], xr[7], xr[8]), x3 = max3_raw(xr[9], xr[10], xr[11]);
        const float x4 = max3_raw(xr[12], xr[13], xr[14]);
        cm = max_raw(max3_raw(x0, x1, x2), max3_raw(x3, x4, xr[15]));
      } else if (pc == 3) {
        const uint32_t u = __float_as_uint(cm);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const float cmax = max_raw(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc2;
        const bool up = cmax > m2 + kLazy;
        mprev = m2;
        m2 = up ? cmax : m2;
        rescale = up;
        nm = (m2 == -INFINITY) ? 0.f : -m2;
      } else {
#pragma unroll
        for (int i = 4 * (pc - 4); i < 4 * (pc - 4) + 4; ++i) p[i] = fast_exp2(fmaf(xr[i], sc2, nm));
      }
    };
    // group g: S MFMA of k-step g for tile i + 1 (past the last tile: a stale
    // slot, result unused), O MFMA (dim tile g / 2, k-step g % 2) for tile
    // i - 1, softmax pieces; LDS operands are read two groups ahead
    f32x16 snext;
#pragma unroll
    for (int e = 0; e < 16; ++e) snext[e] = 0.f;
    bf16x8 kop[3], vop[3];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kop[g] = *reinterpret_cast<const bf16x8*>(kb + kofs[g]);
      if constexpr (kPV) vop[g] = vread(g >> 1, g & 1, vslot);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 2 < NG) {
        kop[(g + 2) % 3] = *reinterpret_cast<const bf16x8*>(kb + kofs[g + 2]);
        if constexpr (kPV) vop[(g + 2) % 3] = vread((g + 2) >> 1, (g + 2) & 1, vslot);
      }
      snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[g % 3], qop[g], snext, 0, 0, 0);
      if constexpr (kPV) oacc[g >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[g % 3], pprev[g & 1], oacc[g >> 1], 0, 0, 0);
#pragma unroll
      for (int pc = g * 8 / NG; pc < (g + 1) * 8 / NG; ++pc) piece(pc);
      // issue order within the group: MFMA, LDS read, 3 VALU, LDS read,
      // 3 VALU, MFMA, LDS read, the rest of the VALU work
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float ps;
    {
      const float s0 = (p[0] + p[1]) + (p[2] + p[3]), s1 = (p[4] + p[5]) + (p[6] + p[7]);
      const float s2v = (p[8] + p[9]) + (p[10] + p[11]), s3 = (p[12] + p[13]) + (p[14] + p[15]);
      ps = (s0 + s1) + (s2v + s3);
    }
    bf16x8 pcur[2];
    pcur[0] = pack_bf16x8(p);
    pcur[1] = pack_bf16x8(p + 8);
    // the rescale by alpha(i) (rare: the reference max moved) follows the
    // accumulation of tile i - 1; its exponential is only taken then
    if (__ballot(rescale)) {
      const float alpha = rescale ? fast_exp2(mprev - m2) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }
    lsum += ps;
    scur = snext;
    pprev[0] = pcur[0];
    pprev[1] = pcur[1];
  };

  if (tid < BQ) cursor[tid] = 0;
  const int kt_first = ts.kmin >> 5, kt_last = ts.kmax >> 5;
  for (int seg0 = kt_first; seg0 <= kt_last; seg0 += SEG) {
    const int nseg = min(SEG, kt_last - seg0 + 1);
    const int key0 = seg0 * 32, key1 = key0 + SEG * 32;
    __syncthreads();
    if (qbits) {
      // the queries' key-membership words (one bit per key, built once per
      // route row by the bitmap pass) are this segment's mask rows as they
      // are: 64 words of one row per direct load, all of a wave's loads in
      // flight together.  Words past the segment (their sources clamped to
      // the row's last word) are never read; rows past the last query are 0.
      const int nch = (nseg + 63) >> 6;
      for (int c = wv; c < BQ * nch; c += 4) {
        const int qi = c / nch, j = ((c - qi * nch) << 6) + lane;
        const int t = qa + qi;
        if (t < a.S_q)
          lds_dma4(qbits + route_row(a, b, t, kvh) * qwords + min(seg0 + j, qwords - 1),
                   __builtin_amdgcn_readfirstlane(lds_addr(&mask[qi][(c - qi * nch) << 6])));
        else
          mask[qi][j] = 0u;
      }
      __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
    } else {
    for (int i = tid; i < BQ * (SEG + 1); i += 256) (&mask[0][0])[i] = 0u;
    __syncthreads();
    // route masks of this segment.  Entry ranges [lo, hi) per query (one lane
    // per query, in parallel): lo is the cursor left by the previous segment,
    // hi the row end when the row's last entry falls in this segment, else a
    // binary search.
    if (wid == 0 && lane < BQ) {
      const int t = qa + lane;
      int lo = cursor[lane], hi = lo;
      if (t < a.S_q) {
        const int n = ts.n_lane;             // min(lens, L) (0 past S_q)
        const int32_t* r = a.routes + route_row(a, b, t, kvh) * a.L;
        // a row's last segment holds all its remaining entries (its last
        // entry, known from the tile statistics, decides), otherwise a
        // binary search
        if (n <= lo || ts.last_lane < key1) {
          hi = max(n, lo);
        } else {
          int l1 = lo, h1 = n;
          while (l1 < h1) { const int m = (l1 + h1) >> 1; if (r[m] < key1) l1 = m + 1; else h1 = m; }
          hi = l1;
        }
      }
      s_lo[lane] = lo;
      s_hi[lane] = hi;
      cursor[lane] = hi;
    }
    __syncthreads();
    // wave w takes queries w, w + 4, ...; each lane takes 8 consecutive
    // entries of a 512-entry chunk.  The route is ascending, so the lane's
    // entries that fall in one mask word are consecutive: their bits are
    // ORed together in registers and the word takes one LDS atomic at the
    // end of the run.  Branch-free: every step issues one atomic, and a step
    // that ends no run (or an entry outside [lo, hi) or the segment) ORs 0
    // into word `lane` of the row -- a different word, and bank, per lane.
    auto or_entries = [&](int qi, int eb, int lo, int hi, const int (&ids)[8]) __attribute__((always_inline)) {
      int wd[8];
      uint32_t bit[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int id = ids[j];
        const bool ok = eb + j >= lo && eb + j < hi && id >= key0 && id < key1 && id < a.S_k;
        const int rel = id - key0;
        wd[j] = ok ? rel >> 5 : -1;
        bit[j] = ok ? 1u << (rel & 31) : 0u;
      }
      uint32_t acc = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc |= bit[j];
        const bool flush = wd[j] >= 0 && (j == 7 || wd[j + 1] != wd[j]);
        atomicOr(&mask[qi][flush ? wd[j] : lane], flush ? acc : 0u);
        acc = (j < 7 && wd[j + 1] == wd[j]) ? acc : 0u;
      }
    };
    if ((a.L & 3) == 0 && a.L >= 4 && (reinterpret_cast<uintptr_t>(a.routes) & 15) == 0) {
      // rows 16-byte aligned: the wave's (query, chunk) items are staged NI at
      // a time in its quarter of the (idle) K/V slots by direct global-to-LDS
      // loads, so their latencies overlap; a chunk starts at the aligned entry
      // below lo, and 16-byte groups past the row end are clamped to its last
      // group (those entries lie beyond hi and are dropped)
      constexpr int QB = 3 * BUF / 4, NI = QB / 2048;
      static_assert(NI >= 1, "route staging");
      const uint32_t wl = lds0 + wv * QB;
      const char* wb = raw + wid * QB;
      int cq = wv, ce = 0;
      if (cq < BQ) ce = __builtin_amdgcn_readfirstlane(s_lo[cq] & ~3);
      while (cq < BQ) {
        int bq[NI], be[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          while (cq < BQ && ce >= s_hi[cq]) {
            cq += 4;
            if (cq < BQ) ce = __builtin_amdgcn_readfirstlane(s_lo[cq] & ~3);
          }
          bq[j] = cq;
          be[j] = ce;
          if (cq < BQ) {
            const int32_t* r = a.routes + route_row(a, b, qa + cq, kvh) * a.L;
#pragma unroll
            for (int h = 0; h < 2; ++h)
              lds_dma16(r + min(ce + 256 * h + 4 * lane, a.L - 4), wl + j * 2048 + h * 1024);
            ce += 512;
          }
        }
        __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
        asm volatile("" : : : "memory");
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if (bq[j] >= BQ) continue;
          const int4 u0 = *reinterpret_cast<const int4*>(wb + j * 2048 + 32 * lane);
          const int4 u1 = *reinterpret_cast<const int4*>(wb + j * 2048 + 32 * lane + 16);
          const int ids[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
          or_entries(bq[j], be[j] + 8 * lane, s_lo[bq[j]], s_hi[bq[j]], ids);
        }
        // the next round overwrites this wave's staging area
        wave_lds_sync();
      }
    } else {
      for (int qi = wid; qi < BQ; qi += 4) {
        const int lo = s_lo[qi], hi = s_hi[qi];
        const int32_t* r = a.routes + route_row(a, b, qa + qi, kvh) * a.L;
        for (int e0 = lo; e0 < hi; e0 += 512) {
          const int eb = e0 + 8 * lane;
          int ids[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) ids[j] = (eb + j < hi) ? r[eb + j] : -1;
          or_entries(qi, eb, lo, hi, ids);
        }
      }
    }
    }
    // every wave's mask words are complete before wave 0 reads them all
    __syncthreads();
    // compact list of the key tiles any query routes to
    if (wid == 0) {
      int base = 0;
      for (int j0 = 0; j0 < SEG; j0 += 64) {
        const int j = j0 + lane;
        uint32_t any = 0u;
        if (j < nseg)
          for (int qi = 0; qi < BQ; ++qi) any |= mask[qi][j];
        const uint64_t bal = __ballot(any != 0u);
        if (any) tiles[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
        base += __popcll(bal);
      }
      if (lane == 0) s_ntiles = base;
    }
    __syncthreads();
    const int ntiles = s_ntiles;
    if (ntiles == 0) continue;
    // prologue: K(0) K(1) K(2) V(0), then S(0)
    issue(seg0 + tiles[0], std::integral_constant<int, 0>{}, KSide{});
    if (ntiles > 1) issue(seg0 + tiles[1], std::integral_constant<int, 1>{}, KSide{});
    if (ntiles > 2) issue(seg0 + tiles[2], std::integral_constant<int, 2>{}, KSide{});
    issue(seg0 + tiles[0], std::integral_constant<int, 0>{}, VSide{});
    if (ntiles > 2) __builtin_amdgcn_s_waitcnt(kDmaWait<2 * NIK + NIV>());
    else if (ntiles > 1) __builtin_amdgcn_s_waitcnt(kDmaWait<NIK + NIV>());
    else __builtin_amdgcn_s_waitcnt(kDmaWait<NIV>());
    bare_barrier();
    nk = tiles[min(3, ntiles - 1)];
    nv = tiles[min(1, ntiles - 1)];
    nmw = mask[colq][tiles[0]];
    scores(scur, 0);
    step(std::integral_constant<int, 0>{}, std::false_type{}, 0, ntiles, seg0);
    // steps 1 .. n - 1, unrolled by three so that every slot offset is a constant
    for (int i = 1; i < ntiles; i += 3) {
      step(std::integral_constant<int, 1>{}, std::true_type{}, i, ntiles, seg0);
      if (i + 1 < ntiles) step(std::integral_constant<int, 2>{}, std::true_type{}, i + 1, ntiles, seg0);
      if (i + 2 < ntiles) step(std::integral_constant<int, 0>{}, std::true_type{}, i + 2, ntiles, seg0);
    }
    // drain: O^T += V^T P^T of the last tile
    __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
    bare_barrier();
    accumulate(pprev, static_cast<uint32_t>((ntiles - 1) % 3) * BUF);
  }

  // ---- epilogue: this lane holds dims 32 dt + 8 j + 4 h32 + {0..3} of its
  // column; the two lane halves together hold the column's row sum
  {
    const int t = qa + colq;
    const uint32_t u = __float_as_uint(lsum);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (kDelta) {
      float part = 0.f;
      if (t < a.S_q) {
        const T* dp = dout + ((static_cast<int64_t>(b) * a.S_q + t) * a.Hq + kvh * G + colh) * DV + 4 * h32;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            part += oacc[dt][e] * inv * bf16_to_f32(dp[32 * dt + 8 * (e >> 2) + (e & 3)]);
      }
      const uint32_t pu = __float_as_uint(part);
      const auto ps = __builtin_amdgcn_permlane32_swap(pu, pu, false, false);
      part = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
      if (t < a.S_q && h32 == 0) delta[(static_cast<int64_t>(b) * a.Hq + kvh * G + colh) * a.S_q + t] = part;
    } else if (t < a.S_q) {
      const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
      T* op = out + (row * a.Hq + kvh * G + colh) * DV + 4 * h32;
      float* o32 = a.o32 ? a.o32 + (row * a.Hq + kvh * G + colh) * DV + 4 * h32 : nullptr;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v[4] = {oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv, oacc[dt][4 * j + 2] * inv,
                              oacc[dt][4 * j + 3] * inv};
          store4(op + 32 * dt + 8 * j, v);
          if (o32) store4(o32 + 32 * dt + 8 * j, v);
        }
      if (h32 == 0)
        lse[(static_cast<int64_t>(b) * a.Hq + kvh * G + colh) * a.S_q + t] = ltot > 0.f ? (m2 + log2f(ltot)) * kLn2 : -INFINITY;
    }
  }
}

// route-density threshold (per mille) above which a query tile runs on the tile kernel
int tile_thr_milli() {
  static int v = [] {
    const char* e = getenv("IRB_TILE_MIN_DENSITY");
    return e ? static_cast<int>(atof(e) * 1000.0) : 120;
  }();
  return v;
}

template <int D, int DV, int G, bool kDelta>
static void launch_tile(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta,
                        const uint32_t* qbits, int qwords, int gather_rest, hipStream_t stream) {
  constexpr int BQ = 128 / G;
  const int n_qt = (a.S_q + BQ - 1) / BQ;
  const unsigned grid = static_cast<unsigned>(a.B) * n_qt * a.Hkv;
  hipLaunchKernelGGL((attn_fwd_tile_kernel<D, DV, G, kDelta>), dim3(grid), dim3(256), 0, stream, a,
                     static_cast<uint16_t*>(out), lse, static_cast<const uint16_t*>(dout), delta, n_qt,
                     tile_thr_milli(), qbits, qwords, gather_rest);
}

// key-membership words per route row, built in the forward's workspace when
// the query-tile kernel can run and they fit the budget (else 0 bytes: the
// tile kernel builds its masks from the routes in LDS)
static constexpr size_t kQbitsBudget = size_t{256} << 20;
size_t attn_fwd_qbits_bytes(const AttnArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (a.dtype != IRB_BF16 || a.Dqk != a.Dv || (a.Dqk != 64 && a.Dqk != 128) || (G != 4 && G != 8 && G != 16)) return 0;
  if (a.S_k > 131072) return 0;
  const size_t words = (static_cast<size_t>(a.S_k) + 31) / 32;
  const size_t bytes = static_cast<size_t>(a.RG) * a.B * a.S_q * words * 4;
  return bytes <= kQbitsBudget ? bytes : 0;
}

template <typename T, int D, int DV, bool kDelta>
static int launch_fwd_t(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int64_t items = static_cast<int64_t>(a.B) * a.S_q * a.Hkv;
  if (items == 0) return 0;
  const int PAD = sizeof(T) == 2 ? 8 : 4;
  const int latent = (a.v == a.k && a.sv_b == a.sk_b && a.sv_t == a.sk_t && a.sv_h == a.sk_h) ? 1 : 0;
  if constexpr (sizeof(T) == 2 && D == 576 && DV == 512) {
    const int rc = launch_latent_fwd(a, out, lse, dout, delta, kDelta, stream);
    if (rc >= 0) return rc;
  }
  int tile_bq = 0;    // > 0: the gather kernel skips the query tiles the tile kernel takes
  if constexpr (sizeof(T) == 2 && (D == 64 || D == 128) && D == DV) {
    // the tile kernel addresses a 32-key tile by 32-bit byte offsets from its first row
    const bool small_strides = static_cast<int64_t>(a.sk_t > a.sv_t ? a.sk_t : a.sv_t) * 64 < (int64_t{1} << 31);
    if (tile_thr_milli() <= 1000 && small_strides && (G == 4 || G == 8 || G == 16)) {
      const size_t qb = attn_fwd_qbits_bytes(a);
      const uint32_t* qbits = nullptr;
      const int qwords = (a.S_k + 31) / 32;
      if (qb > 0 && ws && ws_bytes >= qb) {
        const int64_t rows = static_cast<int64_t>(a.RG) * a.B * a.S_q;
        if (int rc = launch_route_bits(a.routes, a.lens, rows, a.L, a.S_k, static_cast<uint32_t*>(ws), stream)) return rc;
        qbits = static_cast<const uint32_t*>(ws);
      }
      // routes at least thr/1000 of the key range wide: nearly every tile is
      // dense, so the tile launch also gathers the few sparse ones itself and
      // the per-query gather launch (one wave per query just to skip it) is saved
      const bool gather_rest = static_cast<int64_t>(a.L) * 1000 >= static_cast<int64_t>(tile_thr_milli()) * a.S_k;
      if (G == 4) launch_tile<D, DV, 4, kDelta>(a, out, lse, dout, delta, qbits, qwords, gather_rest, stream);
      if (G == 8) launch_tile<D, DV, 8, kDelta>(a, out, lse, dout, delta, qbits, qwords, gather_rest, stream);
      if (G == 16) launch_tile<D, DV, 16, kDelta>(a, out, lse, dout, delta, qbits, qwords, gather_rest, stream);
      if (gather_rest) return 0;
      tile_bq = 128 / G;
    }
  }
  if (G <= 16) {
    const size_t lds = static_cast<size_t>(4) * 32 * (DV + PAD) * sizeof(T);
    auto kern = attn_fwd_kernel<T, D, DV, false, kDelta>;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), lds, stream, a,
                       static_cast<T*>(out), lse, G, static_cast<int>(items), latent, static_cast<const T*>(dout), delta,
                       tile_bq, tile_thr_milli(), gather_head_major(a) ? 1 : 0);
  } else {
    const int slices = (G + 15) / 16;
    const size_t lds = static_cast<size_t>(32) * ((D + PAD) + (latent ? 0 : (DV + PAD))) * sizeof(T);
    auto kern = attn_fwd_kernel<T, D, DV, true, kDelta>;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(items)), dim3(64 * slices), lds, stream, a,
                       static_cast<T*>(out), lse, G, static_cast<int>(items), latent, static_cast<const T*>(dout), delta,
                       0, 0, 0);
  }
  return 0;
}

template <bool kDelta>
static int dispatch_fwd(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (a.dtype == IRB_BF16) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_fwd_t<uint16_t, 64, 64, kDelta>(a, out, lse, dout, delta, ws, ws_bytes, stream);
    if (a.Dqk == 128 && a.Dv == 128) return launch_fwd_t<uint16_t, 128, 128, kDelta>(a, out, lse, dout, delta, ws, ws_bytes, stream);
    if (a.Dqk == 576 && a.Dv == 512) return launch_fwd_t<uint16_t, 576, 512, kDelta>(a, out, lse, dout, delta, ws, ws_bytes, stream);
  } else {
    if (a.Dqk == 64 && a.Dv == 64) return launch_fwd_t<float, 64, 64, kDelta>(a, out, lse, dout, delta, ws, ws_bytes, stream);
    if (a.Dqk == 128 && a.Dv == 128) return launch_fwd_t<float, 128, 128, kDelta>(a, out, lse, dout, delta, ws, ws_bytes, stream);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

int launch_attn_fwd(const AttnArgs& a, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return dispatch_fwd<false>(a, out, lse, nullptr, nullptr, ws, ws_bytes, stream);
}

int launch_attn_delta(const AttnArgs& a, const void* dout, float* delta, hipStream_t stream) {
  return dispatch_fwd<true>(a, nullptr, nullptr, dout, delta, nullptr, 0, stream);
}

}  // namespace irb
