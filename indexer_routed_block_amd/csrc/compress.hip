// a0/a1: document block prefix and key compression (group mean -> RMSNorm -> group-start RoPE).
//
// QSA routing page (nemo_automodel...qwen3_8_flash_next.qsa), indexer class and
// apply_qsa_rope; packed documents per _forward_packed.
//
// One wavefront per compressed block: the c raw rows of the group are read
// with unit-stride lanes over the feature dimension (coalesced), averaged in
// FP32, normalised with a wave reduction and rotated through a per-wave LDS
// staging row (RoPE pairs i and i + D_rope/2 live in different lanes).
#include "irb_internal.hpp"

namespace irb {

constexpr int kMaxDim = 512;        // D_idx upper bound: 8 values per lane
constexpr int kCompressWaves = 4;

// cu_blocks[d] = sum_{d' < d} floor(len_d' / c), d = 0..num_docs.  One
// workgroup; documents handled in chunks of 256 with a running carry.
__global__ void __launch_bounds__(256) cu_blocks_kernel(const int32_t* __restrict__ cu, int num_docs, int c,
                                                        int32_t* __restrict__ cu_blocks) {
  __shared__ int wave_tot[4];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base <= num_docs; base += 256) {
    const int d = base + tid;
    int v = (d < num_docs) ? (cu[d + 1] - cu[d]) / c : 0;
    int incl = wave_incl_scan(v);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int off = carry_s;
    for (int w = 0; w < wid; ++w) off += wave_tot[w];
    if (d <= num_docs) cu_blocks[d] = off + incl - v;   // exclusive prefix
    __syncthreads();
    if (tid == 255) carry_s = off + incl;
    __syncthreads();
  }
}

template <typename T>
__global__ void __launch_bounds__(kCompressWaves * 64)
compress_kernel(Layout L, int c, const T* __restrict__ k, int64_t sb, int64_t st, int D,
                const float* __restrict__ gamma, float eps, const float* __restrict__ freqs, int R,
                const int32_t* __restrict__ cu_blocks, float* __restrict__ kc, int nb_max) {
  __shared__ float stage[kCompressWaves][kMaxDim];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t slot = static_cast<int64_t>(blockIdx.x) * kCompressWaves + wid;
  if (slot >= static_cast<int64_t>(L.B) * nb_max) return;
  const int b = static_cast<int>(slot / nb_max);
  const int j = static_cast<int>(slot % nb_max);
  float* out = kc + slot * D;

  // locate the block: first token of its group, or none (zero slot)
  int first = -1;
  if (L.cu_seqlens) {
    if (j < cu_blocks[L.num_docs]) {
      int lo = 0, hi = L.num_docs - 1;   // largest d with cu_blocks[d] <= j
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_blocks[mid] <= j) lo = mid; else hi = mid - 1;
      }
      first = L.cu_seqlens[lo] + (j - cu_blocks[lo]) * c;
    }
  } else {
    const int n = L.row_lens ? L.row_lens[b] : L.S;
    if (j < n / c) first = j * c;
  }
  const int per = (D + 63) / 64;
  if (first < 0) {
    for (int i = 0; i < per; ++i) {
      const int d = lane + 64 * i;
      if (d < D) out[d] = 0.0f;
    }
    return;
  }

  float m[kMaxDim / 64];
  float ss = 0.0f;
  const T* row0 = k + static_cast<int64_t>(b) * sb + static_cast<int64_t>(first) * st;
#pragma unroll
  for (int i = 0; i < kMaxDim / 64; ++i) {
    m[i] = 0.0f;
    const int d = lane + 64 * i;
    if (i < per && d < D) {
      float s = 0.0f;
      for (int r = 0; r < c; ++r) s += load_as_f32(row0 + static_cast<int64_t>(r) * st + d);
      m[i] = s / static_cast<float>(c);
      ss += m[i] * m[i];
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
  for (int i = 0; i < kMaxDim / 64; ++i) {
    const int d = lane + 64 * i;
    if (i < per && d < D) {
      m[i] = m[i] * inv * gamma[d];
      stage[wid][d] = m[i];
    }
  }
  wave_lds_sync();
  const float* fr = freqs + (static_cast<int64_t>(b) * L.S + first) * R;
  const int half = R / 2;
#pragma unroll
  for (int i = 0; i < kMaxDim / 64; ++i) {
    const int d = lane + 64 * i;
    if (i < per && d < D) {
      float v = m[i];
      if (d < half) {
        v = m[i] * fr[d] - stage[wid][d + half] * fr[half + d];
      } else if (d < R) {
        const int p = d - half;
        v = m[i] * fr[p] + stage[wid][p] * fr[half + p];
      }
      out[d] = v;
    }
  }
}

// bf16 keys with D_idx = D_rope = 128 and c in {4, 8}: lane l holds dims
// 2l, 2l + 1 (one 4-byte load per raw row, all c rows in flight), the RMS
// reduction is a wave sum, and the RoPE partner dims (d +- 64) sit in lane
// l ^ 32, so they come from a cross-lane exchange instead of LDS.
template <int C>
__global__ void __launch_bounds__(kCompressWaves * 64)
compress128_kernel(Layout L, const uint16_t* __restrict__ k, int64_t sb, int64_t st, const float* __restrict__ gamma,
                   float eps, const float* __restrict__ freqs, const int32_t* __restrict__ cu_blocks,
                   float* __restrict__ kc, int nb_max) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t slot = static_cast<int64_t>(blockIdx.x) * kCompressWaves + wid;
  if (slot >= static_cast<int64_t>(L.B) * nb_max) return;
  const int b = static_cast<int>(slot / nb_max);
  const int j = static_cast<int>(slot % nb_max);
  float2* out = reinterpret_cast<float2*>(kc + slot * 128) + lane;
  int first = -1;
  if (L.cu_seqlens) {
    if (j < cu_blocks[L.num_docs]) {
      int lo = 0, hi = L.num_docs - 1;   // largest d with cu_blocks[d] <= j
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_blocks[mid] <= j) lo = mid; else hi = mid - 1;
      }
      first = L.cu_seqlens[lo] + (j - cu_blocks[lo]) * C;
    }
  } else {
    const int n = L.row_lens ? L.row_lens[b] : L.S;
    if (j < n / C) first = j * C;
  }
  if (first < 0) {
    *out = make_float2(0.f, 0.f);
    return;
  }
  const uint16_t* row0 = k + static_cast<int64_t>(b) * sb + static_cast<int64_t>(first) * st + 2 * lane;
  uint32_t raw[C];
#pragma unroll
  for (int r = 0; r < C; ++r) raw[r] = *reinterpret_cast<const uint32_t*>(row0 + static_cast<int64_t>(r) * st);
  const float2 g = reinterpret_cast<const float2*>(gamma)[lane];
  const int p = (2 * lane) & 63;                       // rotary pair index of dim 2l
  const float* fr = freqs + (static_cast<int64_t>(b) * L.S + first) * 128;
  const float2 cs = *reinterpret_cast<const float2*>(fr + p);
  const float2 sn = *reinterpret_cast<const float2*>(fr + 64 + p);
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int r = 0; r < C; ++r) {
    m0 += bf16_to_f32(static_cast<uint16_t>(raw[r] & 0xffffu));
    m1 += bf16_to_f32(static_cast<uint16_t>(raw[r] >> 16));
  }
  m0 /= static_cast<float>(C);
  m1 /= static_cast<float>(C);
  const float ss = wave_sum(m0 * m0 + m1 * m1);
  const float inv = 1.0f / sqrtf(ss / 128.0f + eps);
  m0 = m0 * inv * g.x;
  m1 = m1 * inv * g.y;
  const float o0 = __shfl_xor(m0, 32, 64), o1 = __shfl_xor(m1, 32, 64);
  float2 v;
  if (lane < 32) {   // dims d < 64: u_d cos - u_{d+64} sin
    v.x = m0 * cs.x - o0 * sn.x;
    v.y = m1 * cs.y - o1 * sn.y;
  } else {           // dims d >= 64: u_d cos + u_{d-64} sin
    v.x = m0 * cs.x + o0 * sn.x;
    v.y = m1 * cs.y + o1 * sn.y;
  }
  *out = v;
}

int launch_compress(const Layout& L, int c, const void* k, int dtype, int64_t sb, int64_t st, int D,
                    const float* gamma, float eps, const float* freqs, int R, float* kc,
                    int32_t* cu_blocks, hipStream_t stream) {
  if (L.cu_seqlens) {
    hipLaunchKernelGGL(cu_blocks_kernel, dim3(1), dim3(256), 0, stream, L.cu_seqlens, L.num_docs, c, cu_blocks);
  }
  const int nb_max = L.S / c;
  const int64_t slots = static_cast<int64_t>(L.B) * nb_max;
  if (slots == 0) return 0;
  const dim3 grid(static_cast<unsigned>((slots + kCompressWaves - 1) / kCompressWaves));
  const bool fast = dtype == IRB_BF16 && D == 128 && R == 128 && (c == 4 || c == 8) &&
                    (reinterpret_cast<uintptr_t>(k) & 3) == 0 && (sb % 2) == 0 && (st % 2) == 0 &&
                    (reinterpret_cast<uintptr_t>(freqs) & 7) == 0 && (reinterpret_cast<uintptr_t>(gamma) & 7) == 0;
  if (fast) {
    const uint16_t* kb = static_cast<const uint16_t*>(k);
    if (c == 4)
      hipLaunchKernelGGL(compress128_kernel<4>, grid, dim3(kCompressWaves * 64), 0, stream, L, kb, sb, st, gamma, eps,
                         freqs, cu_blocks, kc, nb_max);
    else
      hipLaunchKernelGGL(compress128_kernel<8>, grid, dim3(kCompressWaves * 64), 0, stream, L, kb, sb, st, gamma, eps,
                         freqs, cu_blocks, kc, nb_max);
    return 0;
  }
  if (dtype == IRB_BF16) {
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, dim3(kCompressWaves * 64), 0, stream, L, c,
                       static_cast<const uint16_t*>(k), sb, st, D, gamma, eps, freqs, R, cu_blocks, kc, nb_max);
  } else {
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kCompressWaves * 64), 0, stream, L, c,
                       static_cast<const float*>(k), sb, st, D, gamma, eps, freqs, R, cu_blocks, kc, nb_max);
  }
  return 0;
}

}  // namespace irb
