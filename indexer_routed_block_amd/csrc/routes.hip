// a4: route expansion (blocks + current tail + window -> ascending token IDs)
// and compaction (arbitrary signed ID rows -> ascending unique valid prefix).
//
// QSA page (nemo_automodel...qwen3_8_flash_next.qsa): select_qsa_token_ids
// (blocks expanded, incomplete-group tail appended, -1 padding),
// qsa_gqa_attention (duplicates collapse); CSA page (step5.sparse),
// RegionMetadata.window_layout (window of the query and W-1 earlier keys);
// latent page (common.cudnn_sparse_attention), _compact_and_sort_indices.
//
// Expansion needs no sort: the selected blocks are ascending and disjoint
// and all lie below the tail, and tail + window form one interval [a, t].
// So the route is "block tokens below a" followed by [a, t]; block tokens
// at or above a are the duplicates.  Every output slot is computed
// independently from its index, so a wavefront writes a route with
// unit-stride, fully coalesced stores.
#include "irb_internal.hpp"

namespace irb {

constexpr int kExpWaves = 4;

// p / c by a multiply-high with m = floor((2^32 - 1) / c) + 1: exact whenever
// p * c < 2^32 (the host checks route width * c); m = 0 means plain division.
IRB_DEV int div_c(int p, int c, uint32_t m) {
  return m ? static_cast<int>(__umulhi(static_cast<uint32_t>(p), m)) : p / c;
}

// One wavefront per query row.  The row's selected blocks are staged in the
// wave's LDS slice (coalesced loads), then every output slot is computed from
// its index; kVec rows (width a multiple of 4, 16-byte aligned) are written
// with 16-byte stores.
template <bool kVec>
__global__ void __launch_bounds__(kExpWaves * 64)
expand_kernel(Layout L, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int topk, int c,
              uint32_t cmagic, int window, const int32_t* __restrict__ cu_blocks, int Lw,
              int32_t* __restrict__ routes, int32_t* __restrict__ lens) {
  extern __shared__ int32_t sblk_all[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kExpWaves + wid;
  if (row >= static_cast<int64_t>(L.B) * L.S) return;
  const int b = static_cast<int>(row / L.S), t = static_cast<int>(row % L.S);
  int32_t* out = routes + row * Lw;
  const Doc d = doc_of(L, b, t);
  if (!d.valid) {
    if constexpr (kVec) {
      for (int p = 4 * lane; p < Lw; p += 256) *reinterpret_cast<int4*>(out + p) = make_int4(-1, -1, -1, -1);
    } else {
      for (int p = lane; p < Lw; p += 64) out[p] = -1;
    }
    if (lane == 0) lens[row] = 0;
    return;
  }
  const int pos = t - d.start;
  const int nb = (pos + 1) / c;
  const int tail0 = d.start + nb * c;                       // first token of the incomplete group
  const int a = window > 0 ? min(tail0, max(d.start, t - window + 1)) : tail0;
  const int base = block_base(L, cu_blocks, d);
  const int k = topk > 0 ? min(max(cnt[row], 0), topk) : 0;   // a caller-supplied count past topk is clamped
  // first token of each selected block, staged in this wave's LDS slice
  int32_t* sb = sblk_all + wid * topk;
  const int32_t* srow = sel + row * topk;
  const int tok0 = d.start - base * c;                      // token of block id x: tok0 + x c
  int full = 0;                                             // blocks whose c tokens all lie below a
#pragma unroll 4
  for (int i = lane; i < k; i += 64) {
    const int s = tok0 + srow[i] * c;
    sb[i] = s;
    full += (s + c <= a) ? 1 : 0;
  }
  full = wave_sum_int(full);
  wave_lds_sync();
  int partial = 0;
  if (full < k) {
    const int s = sb[full];
    if (s < a) partial = a - s;
  }
  const int nblk = full * c + partial;
  const int n = nblk + (t - a + 1);
  auto slot = [&](int p) __attribute__((always_inline)) {
    if (p < nblk) {
      const int i = div_c(p, c, cmagic);
      return sb[i] + (p - i * c);
    }
    return p < n ? a + (p - nblk) : -1;
  };
  if constexpr (kVec) {
    for (int p = 4 * lane; p < Lw; p += 256)
      *reinterpret_cast<int4*>(out + p) = make_int4(slot(p), slot(p + 1), slot(p + 2), slot(p + 3));
  } else {
    for (int p = lane; p < Lw; p += 64) out[p] = slot(p);
  }
  if (lane == 0) lens[row] = n;
}

int launch_expand(const Layout& L, const int32_t* sel, const int32_t* cnt, int topk, int c, int window,
                  const int32_t* cu_blocks, int Lw, int32_t* routes, int32_t* lens, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(L.B) * L.S;
  if (rows == 0) return 0;
  const uint32_t cmagic = (c >= 2 && static_cast<uint64_t>(Lw) * static_cast<uint64_t>(c) < (1ull << 32))
                              ? 0xFFFFFFFFu / static_cast<uint32_t>(c) + 1u
                              : 0u;
  const dim3 grid(static_cast<unsigned>((rows + kExpWaves - 1) / kExpWaves));
  const size_t lds = static_cast<size_t>(kExpWaves) * (topk > 0 ? topk : 1) * sizeof(int32_t);
  const bool vec = (Lw % 4) == 0 && (reinterpret_cast<uintptr_t>(routes) & 15) == 0;
  if (lds > 48 * 1024) {
    const void* fn = vec ? reinterpret_cast<const void*>(expand_kernel<true>) : reinterpret_cast<const void*>(expand_kernel<false>);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
  }
  if (vec)
    hipLaunchKernelGGL(expand_kernel<true>, grid, dim3(kExpWaves * 64), lds, stream, L, sel, cnt, topk, c, cmagic,
                       window, cu_blocks, Lw, routes, lens);
  else
    hipLaunchKernelGGL(expand_kernel<false>, grid, dim3(kExpWaves * 64), lds, stream, L, sel, cnt, topk, c, cmagic,
                       window, cu_blocks, Lw, routes, lens);
  return 0;
}

// ---------------------------------------------------------------- compaction
// One workgroup per row.  When the row's valid IDs span at most kCmpBits
// values (min .. max), they are marked in an LDS bitmap, whose set bits read in
// order are the ascending, duplicate-free prefix (a popcount scan places each
// thread's words).  Wider rows are sorted in LDS (bitonic, invalid IDs as
// INT_MAX) and a block-wide scan of "first of its run" flags writes the
// unique valid prefix in order.
constexpr int kCmpThreads = 256;
constexpr int kCmpBits = 65536;   // bitmap capacity: 8 KiB of LDS

__global__ void __launch_bounds__(kCmpThreads)
compact_kernel(const int32_t* __restrict__ in, int width, int pow2, int64_t key_count, int32_t* __restrict__ out,
               int32_t* __restrict__ lens, int32_t* __restrict__ bad) {
  extern __shared__ int32_t v[];
  __shared__ uint32_t bm[kCmpBits / 32];
  __shared__ int wsum[4];
  __shared__ int s_red[8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t row = blockIdx.x;
  const int32_t* src = in + row * width;
  int32_t* dst = out + row * width;
  int nbad = 0, lo = 0x7fffffff, hi = -1;
  for (int i = tid; i < pow2; i += kCmpThreads) {
    int x = 0x7fffffff;
    if (i < width) {
      const int32_t id = src[i];
      if (id >= 0 && static_cast<int64_t>(id) < key_count) x = id;
      else if (static_cast<int64_t>(id) >= key_count) ++nbad;
    }
    v[i] = x;
    if (x != 0x7fffffff) { lo = min(lo, x); hi = max(hi, x); }
  }
  if (bad) {
    nbad = wave_sum_int(nbad);
    if (lane == 0 && nbad) atomicAdd(bad, nbad);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  if (lane == 0) { s_red[wid] = lo; s_red[4 + wid] = hi; }
  __syncthreads();
  lo = min(min(s_red[0], s_red[1]), min(s_red[2], s_red[3]));
  hi = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));
  int base = 0;
  if (hi < 0) {
    // no valid ID
  } else if (static_cast<int64_t>(hi) - lo < kCmpBits) {
    const int nwords = ((hi - lo) >> 5) + 1;
    for (int i = tid; i < nwords; i += kCmpThreads) bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < width; i += kCmpThreads) {
      const int x = v[i];
      if (x != 0x7fffffff) atomicOr(&bm[(x - lo) >> 5], 1u << ((x - lo) & 31));
    }
    __syncthreads();
    // thread tid owns words [w0, w1): count, scan, then write its IDs into v
    const int wpt = (nwords + kCmpThreads - 1) / kCmpThreads;
    const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
    int cntb = 0;
    for (int w = w0; w < w1; ++w) cntb += __popc(bm[w]);
    int total;
    const int incl = block_scan256(cntb, wsum, &total);
    int pos = incl - cntb;
    for (int w = w0; w < w1; ++w) {
      uint32_t m = bm[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1u;
        v[pos++] = lo + 32 * w + bit;
      }
    }
    base = total;
    __syncthreads();
    for (int i = tid; i < width; i += kCmpThreads) dst[i] = i < base ? v[i] : -1;
  } else {
    for (int k = 2; k <= pow2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < pow2; i += kCmpThreads) {
          const int p = i ^ j;
          if (p > i) {
            const int x = v[i], y = v[p];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { v[i] = y; v[p] = x; }
          }
        }
        __syncthreads();
      }
    }
    for (int i0 = 0; i0 < width; i0 += kCmpThreads) {
      const int i = i0 + tid;
      const int x = (i < width) ? v[i] : 0x7fffffff;
      const int f = (x != 0x7fffffff && (i == 0 || v[i - 1] != x)) ? 1 : 0;
      const int incl_w = wave_incl_scan(f);
      if (lane == 63) wsum[wid] = incl_w;
      __syncthreads();
      int off = 0, tot = 0;
      for (int w2 = 0; w2 < 4; ++w2) { if (w2 < wid) off += wsum[w2]; tot += wsum[w2]; }
      if (f) dst[base + off + incl_w - 1] = x;
      base += tot;
      __syncthreads();
    }
  }
  // the bitmap path wrote the whole row; the others pad the prefix with -1
  const bool whole_row = hi >= 0 && static_cast<int64_t>(hi) - lo < kCmpBits;
  if (!whole_row)
    for (int i = base + tid; i < width; i += kCmpThreads) dst[i] = -1;
  if (tid == 0) lens[row] = base;
}

int launch_compact(const int32_t* in, int64_t rows, int width, int64_t key_count, int32_t* out,
                   int32_t* lens, int32_t* bad, hipStream_t stream) {
  if (rows == 0) return 0;
  int pow2 = 1;
  while (pow2 < width) pow2 <<= 1;
  const size_t lds = static_cast<size_t>(pow2) * sizeof(int32_t);
  hipLaunchKernelGGL(compact_kernel, dim3(static_cast<unsigned>(rows)), dim3(kCmpThreads), lds, stream, in, width,
                     pow2, key_count, out, lens, bad);
  return 0;
}

}  // namespace irb
