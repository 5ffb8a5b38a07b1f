// a3: exact top-k block selection per query row.
//
// QSA page (nemo_automodel...qwen3_8_flash_next.qsa), select_qsa_token_ids:
// the best budget/c visible blocks; CSA page (step5.sparse),
// RegionMetadata.dense_region_ids: with no more than topk visible blocks all
// are taken; RegionSelection.region_ids: ascending IDs, padded.
//
// One workgroup per query row.  The visible scores are turned into
// order-preserving 32-bit keys.  Rows of up to 16384 blocks keep their keys in
// registers (select_reg_kernel): the row's own key range [min, max] is cut
// into 2048 bins, an LDS histogram finds the bin holding the k-th largest key,
// and the bin's range is cut again (11 bits per level, at most three levels)
// until the k-th largest key T itself is known together with how many keys
// equal to T must be taken.  Binning the row's own range, not the keys' top
// bits, spreads the LDS atomics: the top bits of float keys are mostly sign
// and exponent and would send nearly every key to one bin.  Longer rows use
// select_kernel (LDS or global keys, four 8-bit radix passes).  Both emit
// every key > T and the lowest-ID keys == T in block order, so the output is
// ascending without sorting and ties go to the lower block ID.
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
              int32_t* __restrict__ cnt, int hist_only) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ int s_bin, s_above;
  const int tid = threadIdx.x;
  const int r = blockIdx.x, t = q0 + r, b = blockIdx.y;
  int32_t* srow = sel + (static_cast<int64_t>(b) * L.S + t) * topk;
  const Doc d = doc_of(L, b, t);
  const int n = d.valid ? (t - d.start + 1 - hist_only) / c : 0;   // visible blocks (hist: before the query's own)
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

constexpr int kSelBins = 2048;     // bins per level of the register-resident select

// Register-resident select: thread tid holds keys i = 256 e + tid, e < NPT.
template <int NPT>
__global__ void __launch_bounds__(kSelThreads, (NPT >= 64 ? 2 : 4))
select_reg_kernel(Layout L, const float* __restrict__ scores, int64_t stride, int q0, int q1,
                  const int32_t* __restrict__ cu_blocks, int c, int topk, int32_t* __restrict__ sel,
                  int32_t* __restrict__ cnt, int hist_only) {
  static_assert(4 * NPT <= kSelThreads, "one scan entry per (round, wave)");
  __shared__ int hist[kSelBins];
  __shared__ int wsum[4];
  __shared__ uint32_t s_red[8];
  __shared__ int s_bin, s_above;
  __shared__ int s_off[4 * NPT];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x, t = q0 + r, b = blockIdx.y;
  int32_t* srow = sel + (static_cast<int64_t>(b) * L.S + t) * topk;
  const Doc d = doc_of(L, b, t);
  const int n = d.valid ? (t - d.start + 1 - hist_only) / c : 0;   // visible blocks (hist: before the query's own)
  const int base = d.valid ? block_base(L, cu_blocks, d) : 0;
  if (n <= topk) {                     // every visible block is taken
    for (int i = tid; i < topk; i += kSelThreads) srow[i] = (i < n) ? base + i : -1;
    if (tid == 0) cnt[static_cast<int64_t>(b) * L.S + t] = n;
    return;
  }
  const float* row = scores + (static_cast<int64_t>(b) * (q1 - q0) + r) * stride + base;
  // key + 1 (>= 1; +inf gives 0xff800001) for visible blocks, 0 past the row's end:
  // every range and threshold test below then excludes the padding by itself
  // (all loads are issued before the first use: indices clamp to the row's last block)
  float f[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) f[e] = row[min(kSelThreads * e + tid, n - 1)];
  uint32_t key[NPT];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int i = kSelThreads * e + tid;
    key[e] = i < n ? score_key(f[e]) + 1u : 0u;
    kmin = min(kmin, key[e] ? key[e] : 0xffffffffu);
    kmax = max(kmax, key[e]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, 64)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, 64)));
  }
  if (lane == 0) { s_red[wid] = kmin; s_red[4 + wid] = kmax; }
  __syncthreads();
  kmin = min(min(s_red[0], s_red[1]), min(s_red[2], s_red[3]));
  kmax = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));

  // levels: keys k with k - lo <= R fall in bin (k - lo) >> sh (< 2048)
  uint32_t lo = kmin, R = kmax - kmin;
  int sh = max(0, 32 - __clz(static_cast<int>(R)) - 11);
  if (R == 0u) sh = 0;
  int krem = topk;                     // keys still to take inside the current range
  uint32_t T;
  while (true) {
    for (int i = tid; i < kSelBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int i = kSelThreads * e + tid;
      const uint32_t x = key[e] - lo;   // padding (key 0) wraps above R since lo >= 1
      if (x <= R) atomicAdd(&hist[x >> sh], 1);
    }
    __syncthreads();
    // thread tid owns bins 2047 - 8 tid - j (j = 0..7): a scan over threads is
    // a suffix sum over bins
    int h[8], local = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) { h[j] = hist[kSelBins - 1 - 8 * tid - j]; local += h[j]; }
    const int incl = block_incl_scan256(local, wsum);
    if (incl >= krem && incl - local < krem) {
      int acc = incl - local;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (acc >= 0 && acc + h[j] >= krem) { s_bin = kSelBins - 1 - 8 * tid - j; s_above = acc; acc = -1; }
        else if (acc >= 0) acc += h[j];
      }
    }
    __syncthreads();
    const int B = s_bin;
    krem -= s_above;
    lo += static_cast<uint32_t>(B) << sh;
    if (sh == 0) { T = lo; break; }
    R = (1u << sh) - 1u;
    sh = max(0, sh - 11);
    __syncthreads();                   // s_bin / s_above are rewritten by the next level
  }

  // emit in block order: per (round e, wave) counts of keys > T and == T
  const int eq_quota = krem;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const uint64_t bg = __ballot(key[e] > T), be = __ballot(key[e] == T);
    if (lane == 0) s_off[4 * e + wid] = (__popcll(bg) << 16) | __popcll(be);
  }
  __syncthreads();
  const int v = tid < 4 * NPT ? s_off[tid] : 0;
  const int incl = block_incl_scan256(v, wsum);
  if (tid < 4 * NPT) s_off[tid] = incl - v;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int i = kSelThreads * e + tid;
    const int ex = s_off[4 * e + wid];
    const bool gt = key[e] > T, eq = key[e] == T;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int gt_before = (ex >> 16) + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bg >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bg), 0));
    const int eq_before = (ex & 0xffff) + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(be >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(be), 0));
    if (gt || (eq && eq_before < eq_quota)) srow[gt_before + min(eq_before, eq_quota)] = base + i;
  }
  if (tid == 0) cnt[static_cast<int64_t>(b) * L.S + t] = topk;
}

// Rows of at most 64 * NPL blocks: one wavefront per row, NPL keys per lane
// (i = 64 e + lane), 8-bit levels over the row's key range on a per-wave LDS
// histogram and a ballot-based in-order emit; no workgroup barrier at all.
template <int NPL>
__global__ void __launch_bounds__(kSelThreads)
select_wave_kernel(Layout L, const float* __restrict__ scores, int64_t stride, int q0, int q1,
                   const int32_t* __restrict__ cu_blocks, int c, int topk, int32_t* __restrict__ sel,
                   int32_t* __restrict__ cnt, int hist_only) {
  __shared__ int hist_all[kSelThreads / 64][256];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kSelThreads / 64) + wid;
  if (r >= q1 - q0) return;
  const int t = q0 + r, b = blockIdx.y;
  int* hist = hist_all[wid];
  int32_t* srow = sel + (static_cast<int64_t>(b) * L.S + t) * topk;
  const Doc d = doc_of(L, b, t);
  const int n = d.valid ? (t - d.start + 1 - hist_only) / c : 0;   // visible blocks (hist: before the query's own)
  const int base = d.valid ? block_base(L, cu_blocks, d) : 0;
  if (n <= topk) {                     // every visible block is taken
    for (int i = lane; i < topk; i += 64) srow[i] = (i < n) ? base + i : -1;
    if (lane == 0) cnt[static_cast<int64_t>(b) * L.S + t] = n;
    return;
  }
  const float* row = scores + (static_cast<int64_t>(b) * (q1 - q0) + r) * stride + base;
  float f[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) f[e] = row[min(64 * e + lane, n - 1)];
  // key + 1 for visible blocks, 0 past the row's end (excluded by every test below)
  uint32_t key[NPL];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    key[e] = 64 * e + lane < n ? score_key(f[e]) + 1u : 0u;
    kmin = min(kmin, key[e] ? key[e] : 0xffffffffu);
    kmax = max(kmax, key[e]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, 64)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, 64)));
  }
  uint32_t lo = kmin, R = kmax - kmin;
  int sh = R == 0u ? 0 : max(0, 32 - __clz(static_cast<int>(R)) - 8);
  int krem = topk;
  uint32_t T;
  while (true) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[64 * j + lane] = 0;
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      const uint32_t x = key[e] - lo;  // padding (key 0) wraps above R since lo >= 1
      if (x <= R) atomicAdd(&hist[x >> sh], 1);
    }
    wave_lds_sync();
    // lane owns bins 255 - 4 lane - j: a scan over lanes is a suffix sum over bins
    int h[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { h[j] = hist[255 - 4 * lane - j]; local += h[j]; }
    const int incl = wave_incl_scan(local);
    int myb = 0, mya = 0;
    const bool mine = incl >= krem && incl - local < krem;
    if (mine) {
      int acc = incl - local;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (acc >= 0 && acc + h[j] >= krem) { myb = 255 - 4 * lane - j; mya = acc; acc = -1; }
        else if (acc >= 0) acc += h[j];
      }
    }
    const int src = __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
    const int B = __shfl(myb, src, 64);
    krem -= __shfl(mya, src, 64);
    lo += static_cast<uint32_t>(B) << sh;
    if (sh == 0) { T = lo; break; }
    R = (1u << sh) - 1u;
    sh = max(0, sh - 8);
    wave_lds_sync();                   // the histogram is cleared next
  }
  const int eq_quota = krem;
  int gtc = 0, eqc = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const bool gt = key[e] > T, eq = key[e] == T;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int gt_before = gtc + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bg >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bg), 0));
    const int eq_before = eqc + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(be >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(be), 0));
    if (gt || (eq && eq_before < eq_quota)) srow[gt_before + min(eq_before, eq_quota)] = base + 64 * e + lane;
    gtc += __popcll(bg);
    eqc += __popcll(be);
  }
  if (lane == 0) cnt[static_cast<int64_t>(b) * L.S + t] = topk;
}

int launch_select(const Layout& L, const float* scores, int64_t stride, int q0, int q1,
                  const int32_t* cu_blocks, int c, int topk, int32_t* sel, int32_t* cnt,
                  hipStream_t stream, int hist_only) {
  const int n_max = L.S / c;
  const dim3 grid(static_cast<unsigned>(q1 - q0), static_cast<unsigned>(L.B));
#define IRB_SEL_WAVE(NPL)                                                                                  \
  if (n_max <= 64 * NPL) {                                                                                 \
    const dim3 gw(static_cast<unsigned>((q1 - q0 + kSelThreads / 64 - 1) / (kSelThreads / 64)),            \
                  static_cast<unsigned>(L.B));                                                             \
    hipLaunchKernelGGL(select_wave_kernel<NPL>, gw, dim3(kSelThreads), 0, stream, L, scores, stride, q0, q1, \
                       cu_blocks, c, topk, sel, cnt, hist_only);                                                      \
    return 0;                                                                                              \
  }
  IRB_SEL_WAVE(8)
  IRB_SEL_WAVE(16)
  IRB_SEL_WAVE(32)
#undef IRB_SEL_WAVE
#define IRB_SEL_REG(NPT)                                                                                   \
  if (n_max <= kSelThreads * NPT) {                                                                        \
    hipLaunchKernelGGL(select_reg_kernel<NPT>, grid, dim3(kSelThreads), 0, stream, L, scores, stride, q0, q1, \
                       cu_blocks, c, topk, sel, cnt, hist_only);                                                      \
    return 0;                                                                                              \
  }
  IRB_SEL_REG(16)
  IRB_SEL_REG(32)
  IRB_SEL_REG(64)
#undef IRB_SEL_REG
  if (n_max <= kSelMaxLds) {
    const size_t lds = static_cast<size_t>(n_max > 0 ? n_max : 1) * sizeof(uint32_t);
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kSelThreads), lds, stream, L, scores, stride, q0, q1,
                       cu_blocks, c, topk, sel, cnt, hist_only);
  } else {
    hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kSelThreads), 0, stream, L, scores, stride, q0, q1,
                       cu_blocks, c, topk, sel, cnt, hist_only);
  }
  return 0;
}

}  // namespace irb
