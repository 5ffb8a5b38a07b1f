// Step-5 CSA variant of the routing (CSA page, nemo_automodel.components.
// models.step5.sparse): learned region summaries instead of mean-pooled
// blocks, E4M3-rounded scoring inputs, and a selection that always keeps the
// query's current region in an extra slot.
//
//   gather_payload_kernel   gather_region_payload: the keys and compression
//                           logits of every region's source tokens, copied
//                           16 bytes at a time, zeros where a slot is not valid
//   summarize_kernel        _summarize_region_payload (reading): per region
//                           and dimension, the softmax over the valid slots of
//                           the logits weights the keys (FP32), then the sum
//                           is rounded to BF16 and that to E4M3
//   round_e4m3_kernel       E4M3 rounding of index queries (or any tensor) into
//                           bf16 storage
//   region ids              RegionSelection.region_ids: the top-k of the
//                           historical regions (the select kernels with
//                           visibility floor(pos / c)), renumbered so that
//                           every document's regions, its incomplete last
//                           one included, are consecutive, then the current
//                           region, then the sentinel (the region count)
#include <algorithm>

#include "irb_internal.hpp"

namespace irb {

// E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities) round to
// nearest even, as a float: the grid step below |a|'s leading bit is
// 2^(e - 3) for normal exponents e >= -6 and 2^-9 below (subnormals); values
// that round past 448 (to 480) and non-finite values give NaN.  The scaling
// by powers of two is exact, so rintf (ties to even) decides alone.
IRB_DEV float e4m3_rne(float a) {
  if (!(a == a)) return a;
  int e;
  (void)frexpf(a, &e);                        // |a| = m 2^e, 0.5 <= m < 1
  const int lead = max(e - 1, -6);
  const float q = ldexpf(rintf(ldexpf(a, 3 - lead)), lead - 3);
  return fabsf(q) <= 448.f ? q : __int_as_float(0x7fc00000);
}

// 8 elements per thread: one 16-byte output store, 16 (bf16) or 32 (fp32)
// input bytes, when both buffers are 16-byte aligned (vec); element by
// element otherwise and for the tail
__global__ void __launch_bounds__(256)
round_e4m3_kernel(const void* __restrict__ x, int dtype, int64_t n, int vec, uint16_t* __restrict__ out) {
  const int64_t n8 = vec ? n / 8 : 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < n8; g += stride) {
    float v[8];
    if (dtype == IRB_BF16) {
      const uint4 u = reinterpret_cast<const uint4*>(x)[g];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      const float4 a = reinterpret_cast<const float4*>(x)[2 * g];
      const float4 c = reinterpret_cast<const float4*>(x)[2 * g + 1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)        // E4M3 values are exact in bf16
      o[i] = static_cast<uint32_t>(f32_to_bf16(e4m3_rne(v[2 * i]))) |
             (static_cast<uint32_t>(f32_to_bf16(e4m3_rne(v[2 * i + 1]))) << 16);
    reinterpret_cast<uint4*>(out)[g] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  for (int64_t i = 8 * n8 + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const float v = dtype == IRB_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
    out[i] = f32_to_bf16(e4m3_rne(v));
  }
}

// one thread per 16-byte piece of a (slot, row) pair; pieces_per_row = D * esize / 16
__global__ void __launch_bounds__(256)
gather_payload_kernel(const uint4* __restrict__ keys, const uint4* __restrict__ logits, int T, int pieces_per_row,
                      const int32_t* __restrict__ sources, const uint8_t* __restrict__ valid, int64_t slots_per_batch,
                      int64_t n_pieces, uint4* __restrict__ pk, uint4* __restrict__ pz) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_pieces) return;
  const int64_t slot = i / pieces_per_row;
  const int p = static_cast<int>(i - slot * pieces_per_row);
  const int64_t b = slot / slots_per_batch;
  const int src = sources[slot];
  const bool ok = (valid == nullptr || valid[slot] != 0) && src >= 0 && src < T;
  uint4 kv = make_uint4(0u, 0u, 0u, 0u), zv = kv;
  if (ok) {
    const int64_t at = (b * T + src) * pieces_per_row + p;
    kv = keys[at];
    zv = logits[at];
  }
  pk[i] = kv;
  pz[i] = zv;
}

// one thread per (batch, region, dimension); the slots are walked twice (the
// maximum of the valid logits, then the weights and sums), in slot order
template <typename T>
__global__ void __launch_bounds__(256)
summarize_kernel(const T* __restrict__ pk, const T* __restrict__ pz, const uint8_t* __restrict__ valid, int rs,
                 int D, int64_t n, uint16_t* __restrict__ summary) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t reg = i / D;
  const int d = static_cast<int>(i - reg * D);
  const T* kr = pk + reg * rs * D + d;
  const T* zr = pz + reg * rs * D + d;
  const uint8_t* vr = valid + reg * rs;
  float m = -INFINITY;
  for (int s = 0; s < rs; ++s)
    if (vr[s]) m = fmaxf(m, load_as_f32(zr + static_cast<int64_t>(s) * D));
  float den = 0.f, num = 0.f;
  if (m > -INFINITY) {
    for (int s = 0; s < rs; ++s) {
      if (!vr[s]) continue;
      const float e = expf(load_as_f32(zr + static_cast<int64_t>(s) * D) - m);
      den += e;
      num += e * load_as_f32(kr + static_cast<int64_t>(s) * D);
    }
  }
  const float v = den > 0.f ? num / den : 0.f;
  summary[i] = f32_to_bf16(e4m3_rne(bf16_to_f32(f32_to_bf16(v))));
}

// cu_regions[d] = sum_{d' < d} ceil(len_d' / c), d = 0..num_docs (one workgroup, chunks of 256)
__global__ void __launch_bounds__(256)
cu_regions_kernel(const int32_t* __restrict__ cu, int num_docs, int c, int32_t* __restrict__ out) {
  __shared__ int wave_tot[4];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base <= num_docs; base += 256) {
    const int d = base + tid;
    const int v = d < num_docs ? (cu[d + 1] - cu[d] + c - 1) / c : 0;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int off = carry_s;
    for (int w = 0; w < wid; ++w) off += wave_tot[w];
    if (d <= num_docs) out[d] = off + incl - v;
    __syncthreads();
    if (tid == 255) carry_s = off + incl;
    __syncthreads();
  }
}

// rows q0..q1-1: the historical selection `sel` (block ids, ascending, count
// in cnt) renumbered, the current region appended, the sentinel after it;
// cnt becomes the number of used slots
__global__ void __launch_bounds__(256)
region_ids_kernel(Layout L, const int32_t* __restrict__ sel, int32_t* __restrict__ cnt,
                  const int32_t* __restrict__ cu_blocks, const int32_t* __restrict__ cu_regions, int c, int topk,
                  int q0, int q1, int32_t* __restrict__ ids) {
  const int64_t rows = static_cast<int64_t>(L.B) * (q1 - q0);
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int b = static_cast<int>(r / (q1 - q0)), t = q0 + static_cast<int>(r % (q1 - q0));
  const int64_t row = static_cast<int64_t>(b) * L.S + t;
  const Doc d = doc_of(L, b, t);
  int total;
  if (L.cu_seqlens) total = cu_regions[L.num_docs];
  else total = ((L.row_lens ? L.row_lens[b] : L.S) + c - 1) / c;
  int32_t* out = ids + row * (topk + 1);
  const int k = d.valid ? min(max(cnt[row], 0), topk) : 0;
  const int rb = L.cu_seqlens ? cu_regions[d.index] : 0;
  const int bb = block_base(L, cu_blocks, d);
  const int cur = rb + (t - d.start) / c;
  for (int i = lane; i <= topk; i += 64) {
    int v = total;
    if (d.valid) {
      if (i < k) v = rb + (sel[row * topk + i] - bb);
      else if (i == k) v = cur;
    }
    out[i] = v;
  }
  if (lane == 0) cnt[row] = d.valid ? k + 1 : 0;
}

int launch_round_e4m3(const void* x, int dtype, int64_t n, uint16_t* out, hipStream_t stream) {
  if (n <= 0) return 0;
  const int vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 ? 1 : 0;
  const int64_t per = vec ? 8 : 1;
  const int64_t blocks = std::min<int64_t>((n + 256 * per - 1) / (256 * per), 65536);
  hipLaunchKernelGGL(round_e4m3_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, x, dtype, n, vec,
                     out);
  return 0;
}

int launch_gather_payload(const void* keys, const void* logits, int esize, int B, int T, int D, const int32_t* sources,
                          const uint8_t* valid, int R, int rs, void* pk, void* pz, hipStream_t stream) {
  const int ppr = D * esize / 16;
  const int64_t n = static_cast<int64_t>(B) * R * rs * ppr;
  if (n == 0) return 0;
  hipLaunchKernelGGL(gather_payload_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint4*>(keys), static_cast<const uint4*>(logits), T, ppr, sources, valid,
                     static_cast<int64_t>(R) * rs, n, static_cast<uint4*>(pk), static_cast<uint4*>(pz));
  return 0;
}

int launch_summarize(const void* pk, const void* pz, int dtype, const uint8_t* valid, int B, int R, int rs, int D,
                     uint16_t* summary, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(B) * R * D;
  if (n == 0) return 0;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (dtype == IRB_BF16)
    hipLaunchKernelGGL(summarize_kernel<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(pk),
                       static_cast<const uint16_t*>(pz), valid, rs, D, n, summary);
  else
    hipLaunchKernelGGL(summarize_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(pk),
                       static_cast<const float*>(pz), valid, rs, D, n, summary);
  return 0;
}

size_t region_ids_workspace_bytes(int B, int S, int topk, int num_docs) {
  return (static_cast<size_t>(B) * S * topk * 4 + 255) / 256 * 256 + static_cast<size_t>(num_docs + 1) * 4;
}

int launch_region_ids(const Layout& L, const float* scores, int64_t stride, int q0, int q1, const int32_t* cu_blocks,
                      int c, int topk, int32_t* ids, int32_t* cnt, void* ws, hipStream_t stream) {
  int32_t* sel = static_cast<int32_t*>(ws);
  int32_t* cu_regions = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                   (static_cast<size_t>(L.B) * L.S * topk * 4 + 255) / 256 * 256);
  if (int rc = launch_select(L, scores, stride, q0, q1, cu_blocks, c, topk, sel, cnt, stream, 1)) return rc;
  if (L.cu_seqlens)
    hipLaunchKernelGGL(cu_regions_kernel, dim3(1), dim3(256), 0, stream, L.cu_seqlens, L.num_docs, c, cu_regions);
  const int64_t rows = static_cast<int64_t>(L.B) * (q1 - q0);
  hipLaunchKernelGGL(region_ids_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, L, sel,
                     cnt, cu_blocks, cu_regions, c, topk, q0, q1, ids);
  return 0;
}

}  // namespace irb
