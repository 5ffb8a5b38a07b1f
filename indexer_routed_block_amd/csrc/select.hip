// a3: exact top-k block selection per query row.
//
// QSA page (nemo_automodel...qwen3_8_flash_next.qsa), select_qsa_token_ids:
// the best budget/c visible blocks; CSA page (step5.sparse),
// RegionMetadata.dense_region_ids: with no more than topk visible blocks all
// are taken; RegionSelection.region_ids: ascending IDs, padded.
//
// One workgroup per query row.  The visible scores are turned into
// order-preserving 32-bit keys and kept in LDS.  A 4-pass radix select (8-bit
// digits, LDS histograms) finds the k-th largest key T and how many keys
// equal to T must be taken.  A final in-order pass over 256-key rounds emits
// every key > T and the lowest-ID keys == T, so the output is ascending
// without sorting and ties go to the lower block ID.
#include "irb_internal.hpp"

namespace irb {

constexpr int kSelThreads = 256;
constexpr int kSelMaxLds = 32768;   // keys kept in LDS (128 KiB); longer rows re-read global memory

// inclusive scan over the 256 threads of a workgroup; wsum is 4 ints of LDS
IRB_DEV int block_incl_scan256(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int off = 0;
  for (int w2 = 0; w2 < wid; ++w2) off += wsum[w2];
  __syncthreads();
  return incl + off;
}

template <bool kInLds>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(Layout L, const float* __restrict__ scores, int64_t stride, int q0, int q1,
              const int32_t* __restrict__ cu_blocks, int c, int topk, int32_t* __restrict__ sel,
              int32_t* __restrict__ cnt) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ int s_bin, s_above;
  const int tid = threadIdx.x;
  const int r = blockIdx.x, t = q0 + r, b = blockIdx.y;
  int32_t* srow = sel + (static_cast<int64_t>(b) * L.S + t) * topk;
  const Doc d = doc_of(L, b, t);
  const int n = d.valid ? (t - d.start + 1) / c : 0;
  const int base = d.valid ? block_base(L, cu_blocks, d) : 0;
  if (n <= topk) {                     // every visible block is taken
    for (int i = tid; i < topk; i += kSelThreads) srow[i] = (i < n) ? base + i : -1;
    if (tid == 0) cnt[static_cast<int64_t>(b) * L.S + t] = n;
    return;
  }
  const float* row = scores + (static_cast<int64_t>(b) * (q1 - q0) + r) * stride + base;
  if (kInLds) {
    for (int i = tid; i < n; i += kSelThreads) keys[i] = score_key(row[i]);
    __syncthreads();
  }
  auto key_at = [&](int i) -> uint32_t { return kInLds ? keys[i] : score_key(row[i]); };

  uint32_t prefix = 0, mask = 0;
  int krem = topk;                     // keys still to take at and below the current prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    // thread tid holds bin 255-tid: a prefix scan over threads is a suffix sum over bins
    const int v = hist[255 - tid];
    const int incl = block_incl_scan256(v, wsum);
    if (incl >= krem && incl - v < krem) { s_bin = 255 - tid; s_above = incl - v; }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_bin) << shift;
    mask |= 255u << shift;
    krem -= s_above;
    __syncthreads();
  }
  // prefix == T, the k-th largest key; krem keys equal to T are taken (lowest IDs first)
  const uint32_t T = prefix;
  int out_base = 0, eq_quota = krem;
  for (int i0 = 0; i0 < n; i0 += kSelThreads) {
    const int i = i0 + tid;
    const uint32_t k = (i < n) ? key_at(i) : 0u;
    const int gt = (i < n && k > T) ? 1 : 0;
    const int eq = (i < n && k == T) ? 1 : 0;
    const int packed = (gt << 16) | eq;
    const int incl = block_incl_scan256(packed, wsum);
    const int ex = incl - packed;
    const int gt_ex = ex >> 16, eq_ex = ex & 0xffff;
    if (gt || (eq && eq_ex < eq_quota)) srow[out_base + gt_ex + min(eq_ex, eq_quota)] = base + i;
    // totals of the round are the last thread's inclusive values
    if (tid == kSelThreads - 1) { wsum[0] = incl >> 16; wsum[1] = incl & 0xffff; }
    __syncthreads();
    const int gt_tot = wsum[0], eq_tot = wsum[1];
    __syncthreads();
    const int eq_take = min(eq_tot, eq_quota);
    out_base += gt_tot + eq_take;
    eq_quota -= eq_take;
  }
  if (tid == 0) cnt[static_cast<int64_t>(b) * L.S + t] = topk;
}

int launch_select(const Layout& L, const float* scores, int64_t stride, int q0, int q1,
                  const int32_t* cu_blocks, int c, int topk, int32_t* sel, int32_t* cnt,
                  hipStream_t stream) {
  const int n_max = L.S / c;
  const dim3 grid(static_cast<unsigned>(q1 - q0), static_cast<unsigned>(L.B));
  if (n_max <= kSelMaxLds) {
    const size_t lds = static_cast<size_t>(n_max > 0 ? n_max : 1) * sizeof(uint32_t);
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kSelThreads), lds, stream, L, scores, stride, q0, q1,
                       cu_blocks, c, topk, sel, cnt);
  } else {
    hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kSelThreads), 0, stream, L, scores, stride, q0, q1,
                       cu_blocks, c, topk, sel, cnt);
  }
  return 0;
}

}  // namespace irb
