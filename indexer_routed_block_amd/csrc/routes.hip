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

__global__ void __launch_bounds__(kExpWaves * 64)
expand_kernel(Layout L, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, int topk, int c,
              int window, const int32_t* __restrict__ cu_blocks, int Lw, int32_t* __restrict__ routes,
              int32_t* __restrict__ lens) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kExpWaves + wid;
  if (row >= static_cast<int64_t>(L.B) * L.S) return;
  const int b = static_cast<int>(row / L.S), t = static_cast<int>(row % L.S);
  int32_t* out = routes + row * Lw;
  const Doc d = doc_of(L, b, t);
  if (!d.valid) {
    for (int p = lane; p < Lw; p += 64) out[p] = -1;
    if (lane == 0) lens[row] = 0;
    return;
  }
  const int pos = t - d.start;
  const int nb = (pos + 1) / c;
  const int tail0 = d.start + nb * c;                       // first token of the incomplete group
  const int a = window > 0 ? min(tail0, max(d.start, t - window + 1)) : tail0;
  const int base = block_base(L, cu_blocks, d);
  const int k = cnt[row];
  const int32_t* srow = sel + row * topk;
  // blocks whose c tokens all lie below a (a prefix of the ascending list)
  int full = 0;
  for (int i = lane; i < k; i += 64) full += (d.start + (srow[i] - base) * c + c <= a) ? 1 : 0;
  full = wave_sum_int(full);
  int partial = 0;
  if (full < k) {
    const int s = d.start + (srow[full] - base) * c;
    if (s < a) partial = a - s;
  }
  const int nblk = full * c + partial;
  const int n = nblk + (t - a + 1);
  for (int p = lane; p < Lw; p += 64) {
    int v = -1;
    if (p < nblk) {
      const int i = p / c;
      v = d.start + (srow[i] - base) * c + (p - i * c);
    } else if (p < n) {
      v = a + (p - nblk);
    }
    out[p] = v;
  }
  if (lane == 0) lens[row] = n;
}

int launch_expand(const Layout& L, const int32_t* sel, const int32_t* cnt, int topk, int c, int window,
                  const int32_t* cu_blocks, int Lw, int32_t* routes, int32_t* lens, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(L.B) * L.S;
  if (rows == 0) return 0;
  hipLaunchKernelGGL(expand_kernel, dim3(static_cast<unsigned>((rows + kExpWaves - 1) / kExpWaves)),
                     dim3(kExpWaves * 64), 0, stream, L, sel, cnt, topk, c, window, cu_blocks, Lw, routes, lens);
  return 0;
}

// ---------------------------------------------------------------- compaction
// One workgroup per row: bitonic sort of the row (invalid IDs as INT_MAX) in
// LDS, then a block-wide scan of "first of its run" flags writes the unique
// valid prefix in order.
constexpr int kCmpThreads = 256;

__global__ void __launch_bounds__(kCmpThreads)
compact_kernel(const int32_t* __restrict__ in, int width, int pow2, int64_t key_count, int32_t* __restrict__ out,
               int32_t* __restrict__ lens, int32_t* __restrict__ bad) {
  extern __shared__ int32_t v[];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int32_t* src = in + row * width;
  int nbad = 0;
  for (int i = tid; i < pow2; i += kCmpThreads) {
    int x = 0x7fffffff;
    if (i < width) {
      const int32_t id = src[i];
      if (id >= 0 && static_cast<int64_t>(id) < key_count) x = id;
      else if (static_cast<int64_t>(id) >= key_count) ++nbad;
    }
    v[i] = x;
  }
  __syncthreads();
  if (bad) {
    nbad = wave_sum_int(nbad);
    if ((tid & 63) == 0 && nbad) atomicAdd(bad, nbad);
  }
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
  int32_t* dst = out + row * width;
  int base = 0;
  for (int i0 = 0; i0 < width; i0 += kCmpThreads) {
    const int i = i0 + tid;
    const int x = (i < width) ? v[i] : 0x7fffffff;
    const int f = (x != 0x7fffffff && (i == 0 || v[i - 1] != x)) ? 1 : 0;
    const int wl = tid & 63, wid = tid >> 6;
    const int incl_w = wave_incl_scan(f);
    if (wl == 63) wsum[wid] = incl_w;
    __syncthreads();
    int off = 0, tot = 0;
    for (int w2 = 0; w2 < 4; ++w2) { if (w2 < wid) off += wsum[w2]; tot += wsum[w2]; }
    if (f) dst[base + off + incl_w - 1] = x;
    base += tot;
    __syncthreads();
  }
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
