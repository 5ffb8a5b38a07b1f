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
template <typename T, int D, int DV, bool kShared, bool kDelta>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(AttnArgs a, T* __restrict__ out, float* __restrict__ lse, int G, int n_items, int latent,
                const T* __restrict__ dout, float* __restrict__ delta) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int KS = D / 32;
  constexpr int NDT = DV / 16;
  constexpr int PAD = sizeof(T) == 2 ? 8 : 4;
  constexpr int LDK = D + PAD;
  constexpr int LDV = DV + PAD;
  extern __shared__ __align__(16) char smem[];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  int item, slice;
  if (kShared) {
    item = blockIdx.x;
    slice = wid;
  } else {
    item = blockIdx.x * 4 + wid;
    slice = 0;
    if (item >= n_items) return;
  }
  const int kvh = item % a.Hkv;
  const int t = (item / a.Hkv) % a.S_q;
  const int b = item / (a.Hkv * a.S_q);
  const int h0 = kvh * G + 16 * slice;
  const int nh = min(16, G - 16 * slice);
  const T* qbase = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t;
  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int n = max(0, min(a.lens[row], a.L));
  const int32_t* route = a.routes + row * a.L;

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
    vl = reinterpret_cast<T*>(smem) + wid * 32 * LDV;
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
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float mnew = fmaxf(m2, cmax);
    float alpha = 1.f;
    float p[2][4];
    if (mnew == -INFINITY) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[ti][i] = 0.f;
    } else {
      alpha = exp2f(m2 - mnew);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[ti][i] = exp2f(x[ti][i] - mnew);
    }
    m2 = mnew;
    float ps = 0.f;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) ps += p[ti][i];
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;

    // P^T operand: k positions 8*g16 + j <-> keys {4g..4g+3} of tile 0, then of tile 1
    bf16x8 ph, pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      put_p(ph, pl, j, p[0][j], kSplit);
      put_p(ph, pl, 4 + j, p[1][j], kSplit);
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

  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
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
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (l16 < nh && g16 == 0) delta[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = part;
    return;
  }
  if (l16 < nh) {
    T* op = out + (row * a.Hq + h0 + l16) * DV + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float v[4] = {oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv};
      store4(op + dt * 16, v);
    }
    if (g16 == 0)
      lse[(static_cast<int64_t>(b) * a.Hq + h0 + l16) * a.S_q + t] = ltot > 0.f ? (m2 + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, int DV, bool kDelta>
static int launch_fwd_t(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int64_t items = static_cast<int64_t>(a.B) * a.S_q * a.Hkv;
  if (items == 0) return 0;
  const int PAD = sizeof(T) == 2 ? 8 : 4;
  const int latent = (a.v == a.k && a.sv_b == a.sk_b && a.sv_t == a.sk_t && a.sv_h == a.sk_h) ? 1 : 0;
  if (G <= 16) {
    const size_t lds = static_cast<size_t>(4) * 32 * (DV + PAD) * sizeof(T);
    auto kern = attn_fwd_kernel<T, D, DV, false, kDelta>;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), lds, stream, a,
                       static_cast<T*>(out), lse, G, static_cast<int>(items), latent, static_cast<const T*>(dout), delta);
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
                       static_cast<T*>(out), lse, G, static_cast<int>(items), latent, static_cast<const T*>(dout), delta);
  }
  return 0;
}

template <bool kDelta>
static int dispatch_fwd(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, hipStream_t stream) {
  if (a.dtype == IRB_BF16) {
    if (a.Dqk == 64 && a.Dv == 64) return launch_fwd_t<uint16_t, 64, 64, kDelta>(a, out, lse, dout, delta, stream);
    if (a.Dqk == 128 && a.Dv == 128) return launch_fwd_t<uint16_t, 128, 128, kDelta>(a, out, lse, dout, delta, stream);
    if (a.Dqk == 576 && a.Dv == 512) return launch_fwd_t<uint16_t, 576, 512, kDelta>(a, out, lse, dout, delta, stream);
  } else {
    if (a.Dqk == 64 && a.Dv == 64) return launch_fwd_t<float, 64, 64, kDelta>(a, out, lse, dout, delta, stream);
    if (a.Dqk == 128 && a.Dv == 128) return launch_fwd_t<float, 128, 128, kDelta>(a, out, lse, dout, delta, stream);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

int launch_attn_fwd(const AttnArgs& a, void* out, float* lse, hipStream_t stream) {
  return dispatch_fwd<false>(a, out, lse, nullptr, nullptr, stream);
}

int launch_attn_delta(const AttnArgs& a, const void* dout, float* delta, hipStream_t stream) {
  return dispatch_fwd<true>(a, nullptr, nullptr, dout, delta, stream);
}

}  // namespace irb
