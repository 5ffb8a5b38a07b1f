// a5: forward (query tile -> key tiles) and reverse (key tile -> query tiles)
// block lists from token routes.
//
// FA4 page (nemo_automodel...step5.fa4): _block_lists (no dense grid),
// _selected_block_lists (route-derived forward/reverse lists with bounded
// scratch), _BackwardBlockPartition (counts + ascending padded indices).
//
// Two passes over a bit matrix in caller-provided scratch (1 bit per
// (row tile, other-axis tile) pair).  Mark: a wavefront reads a query's route
// (coalesced, 64 or 256 entries per step) and sets the bit of every new tile
// once per run of equal tiles -- for reverse lists into a band of the matrix
// held in LDS by the workgroup that owns the band's query tiles, written out
// whole afterwards; otherwise (forward lists, or key-tile counts whose band
// would not fit in LDS) by global atomics into the zeroed matrix.  Emit: a
// workgroup scans one row with popcount prefix sums and writes the ascending
// tile list and its -1 padding.
#include "irb_internal.hpp"

namespace irb {

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

int launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p, n, v);
  return 0;
}

constexpr int kMarkWaves = 4;

// id / bk by a multiply-high with m = floor((2^32 - 1) / bk) + 1, exact for
// id * bk < 2^32 (the host checks S_k * bk); m = 0 means plain division
IRB_DEV int div_bk(int id, int bk, uint32_t m) {
  return m ? static_cast<int>(__umulhi(static_cast<uint32_t>(id), m)) : id / bk;
}

// Walks one ascending route (n entries at r, in a row of w entries) with a
// whole wavefront and calls mark(kt) once per run of equal key tiles
// kt = id / bk.  kVec rows (w a multiple of 4, 16-byte aligned) are read four
// entries per lane per load, four 256-entry chunks in flight.  Out-of-range
// IDs are ignored.
template <bool kVec, typename Mark>
IRB_DEV void walk_route_tiles(const int32_t* __restrict__ r, int n, int w, int S_k, int bk, uint32_t bkm, Mark&& mark) {
  const int lane = threadIdx.x & 63;
  int prev_last = -1;
  if constexpr (kVec) {
    if (n <= 0) return;
    // chunk c + 4 is loaded when chunk c is marked: the loop is unrolled by
    // four over fixed register slots and every load is issued (addresses past
    // the row clamped to its last four entries), with no exit inside the
    // unrolled body, so the waits stay counted; entries past n, including
    // whole chunks after the last, are ignored
    constexpr int PF = 4;
    auto ld = [&](int e) __attribute__((always_inline)) { return *reinterpret_cast<const int4*>(r + min(e, w - 4)); };
    int4 slot[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) slot[p] = ld(256 * p + 4 * lane);
    for (int e00 = 0; e00 < n; e00 += 256 * PF)
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int e0 = e00 + 256 * p;
      const int e = e0 + 4 * lane;
      const int4 v = slot[p];
      slot[p] = ld(e + 256 * PF);
      const int ids[4] = {v.x, v.y, v.z, v.w};
      int kt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = e + j < n && ids[j] >= 0 && ids[j] < S_k;
        kt[j] = ok ? div_bk(ids[j], bk, bkm) : -1;
      }
      int before = __shfl_up(kt[3], 1, 64);
      if (lane == 0) before = prev_last;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kt[j] >= 0 && kt[j] != before) mark(kt[j]);
        if (kt[j] >= 0) before = kt[j];
      }
      // a tile already marked for the next chunk's first entry: the largest
      // of the highest lane holding a valid entry (the route is ascending)
      const int lmax = max(max(kt[0], kt[1]), max(kt[2], kt[3]));
      const uint64_t bal = __ballot(lmax >= 0);
      if (bal) prev_last = max(prev_last, __builtin_amdgcn_readlane(lmax, 63 - __builtin_clzll(bal)));
    }
  } else {
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + lane;
      const int id = (e < n) ? r[e] : -1;
      const bool ok = id >= 0 && id < S_k;
      const int kt = ok ? div_bk(id, bk, bkm) : -1;
      int before = __shfl_up(kt, 1, 64);
      if (lane == 0) before = prev_last;
      if (ok && kt != before) mark(kt);
      prev_last = max(prev_last, wave_max_int(kt));
    }
  }
}

// One wavefront per query row (b, t); one global atomic OR per run of equal
// tiles into the zeroed bit matrix.
template <bool kVec>
__global__ void __launch_bounds__(kMarkWaves * 64)
mark_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ lens, int B, int S_q, int S_k, int Lw,
            int bq, int bk, uint32_t bkm, int reverse, int n_rows, int words, uint32_t* __restrict__ bits) {
  const int wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kMarkWaves + wid;
  if (row >= static_cast<int64_t>(B) * S_q) return;
  const int b = static_cast<int>(row / S_q), t = static_cast<int>(row % S_q);
  const int n = max(0, min(lens[row], Lw));
  const int qt = t / bq;
  uint32_t* mat = bits + static_cast<int64_t>(b) * n_rows * words;
  walk_route_tiles<kVec>(routes + row * Lw, n, Lw, S_k, bk, bkm, [&](int kt) __attribute__((always_inline)) {
    if (reverse) atomicOr(&mat[static_cast<int64_t>(kt) * words + (qt >> 5)], 1u << (qt & 31));
    else atomicOr(&mat[static_cast<int64_t>(qt) * words + (kt >> 5)], 1u << (kt & 31));
  });
}

// Reverse lists: one workgroup per band of qw consecutive words (32 qw query
// tiles) of one batch row.  The band's words of every key-tile row are built
// in LDS with LDS atomics (wave w walks the band's queries w, w + 8, ...),
// then every word of the band is written out, zeros included, so the matrix
// needs neither a clearing pass nor global atomics.
constexpr int kBandWaves = 8;

template <bool kVec>
__global__ void __launch_bounds__(kBandWaves * 64)
mark_band_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ lens, int S_q, int S_k, int Lw,
                 int bq, int bk, uint32_t bkm, int n_rows, int words, int qw, uint32_t* __restrict__ bits) {
  extern __shared__ uint32_t band[];   // [n_rows][qw]
  const int tid = threadIdx.x, wid = tid >> 6;
  const int b = blockIdx.y;
  const int w0 = blockIdx.x * qw;
  const int nw = min(qw, words - w0);
  for (int i = tid; i < n_rows * qw; i += kBandWaves * 64) band[i] = 0u;
  __syncthreads();
  const int qt0 = 32 * w0;
  const int t1 = static_cast<int>(min(static_cast<int64_t>(S_q), static_cast<int64_t>(qt0 + 32 * nw) * bq));
  for (int t = qt0 * bq + wid; t < t1; t += kBandWaves) {
    const int64_t row = static_cast<int64_t>(b) * S_q + t;
    const int n = max(0, min(lens[row], Lw));
    const int rel = t / bq - qt0;
    uint32_t* col = band + (rel >> 5);
    const uint32_t bit = 1u << (rel & 31);
    walk_route_tiles<kVec>(routes + row * Lw, n, Lw, S_k, bk, bkm,
                           [&](int kt) __attribute__((always_inline)) { atomicOr(&col[kt * qw], bit); });
  }
  __syncthreads();
  uint32_t* mat = bits + static_cast<int64_t>(b) * n_rows * words + w0;
  for (int i = tid; i < n_rows * qw; i += kBandWaves * 64) {
    const int kt = i / qw, j = i - kt * qw;
    if (j < nw) mat[static_cast<int64_t>(kt) * words + j] = band[i];
  }
}

// One workgroup per bit-matrix row: popcount prefix sums over the row's
// words (four per thread per step when vec_in), the ascending list, then -1
// up to the row's width (16-byte stores when vec_out).
__global__ void __launch_bounds__(256)
emit_kernel(const uint32_t* __restrict__ bits, int n_rows, int words, int32_t* __restrict__ counts,
            int32_t* __restrict__ indices, int width, int vec_in, int vec_out) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int b = blockIdx.y, row = blockIdx.x;
  const uint32_t* w = bits + (static_cast<int64_t>(b) * n_rows + row) * words;
  int32_t* out = indices + (static_cast<int64_t>(b) * n_rows + row) * width;
  int base = 0;
  if (vec_in) {
    for (int w0 = 0; w0 < words; w0 += 1024) {
      const int i = w0 + 4 * tid;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (i < words) x = *reinterpret_cast<const uint4*>(w + i);
      const int pc = __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
      int tot;
      const int incl = block_scan256(pc, wsum, &tot);
      int o = base + incl - pc;
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t y = xs[j];
        while (y) {
          const int bit = __ffs(y) - 1;
          y &= y - 1;
          out[o++] = (i + j) * 32 + bit;
        }
      }
      base += tot;
    }
  } else {
    for (int w0 = 0; w0 < words; w0 += 256) {
      const int i = w0 + tid;
      const uint32_t x = (i < words) ? w[i] : 0u;
      const int pc = __popc(x);
      int tot;
      const int incl = block_scan256(pc, wsum, &tot);
      int o = base + incl - pc;
      uint32_t y = x;
      while (y) {
        const int bit = __ffs(y) - 1;
        y &= y - 1;
        out[o++] = i * 32 + bit;
      }
      base += tot;
    }
  }
  if (vec_out) {
    const int a = min(width, (base + 3) & ~3);
    if (base + tid < a) out[base + tid] = -1;
    for (int i = a + 4 * tid; i < width; i += 1024) *reinterpret_cast<int4*>(out + i) = make_int4(-1, -1, -1, -1);
  } else {
    for (int i = base + tid; i < width; i += 256) out[i] = -1;
  }
  if (tid == 0) counts[static_cast<int64_t>(b) * n_rows + row] = base;
}

// words per band of the reverse-list mark (0: the atomic path).  A band's
// LDS (n_rows x qw words) stays within 64 KiB, two workgroups per CU, and
// qw shrinks until the grid has at least 1024 bands.
static int band_words(int B, int n_rows, int words) {
  int qw = 8;
  while (qw > 1 && (static_cast<int64_t>(n_rows) * qw * 4 > 65536 ||
                    static_cast<int64_t>(B) * ((words + qw - 1) / qw) < 1024))
    qw >>= 1;
  return static_cast<int64_t>(n_rows) * qw * 4 <= 65536 ? qw : 0;
}

int launch_block_lists(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int Lw, int bq, int bk,
                       int reverse, int32_t* counts, int32_t* indices, int width, uint32_t* bitmap,
                       hipStream_t stream) {
  const int nqt = (S_q + bq - 1) / bq, nkt = (S_k + bk - 1) / bk;
  const int n_rows = reverse ? nkt : nqt;
  const int n_other = reverse ? nqt : nkt;
  const int words = (n_other + 31) / 32;
  const int64_t qrows = static_cast<int64_t>(B) * S_q;
  const uint32_t bkm = (bk >= 2 && static_cast<uint64_t>(S_k) * static_cast<uint64_t>(bk) < (1ull << 32))
                           ? 0xFFFFFFFFu / static_cast<uint32_t>(bk) + 1u
                           : 0u;
  const bool vec_routes = (Lw % 4) == 0 && (reinterpret_cast<uintptr_t>(routes) & 15) == 0;
  const int qw = reverse ? band_words(B, n_rows, words) : 0;
  if (qw > 0) {
    // every word of the matrix is written by exactly one band
    const dim3 grid(static_cast<unsigned>((words + qw - 1) / qw), static_cast<unsigned>(B));
    const size_t lds = static_cast<size_t>(n_rows) * qw * 4;
    if (vec_routes)
      hipLaunchKernelGGL(mark_band_kernel<true>, grid, dim3(kBandWaves * 64), lds, stream, routes, lens, S_q, S_k, Lw, bq, bk, bkm,
                         n_rows, words, qw, bitmap);
    else
      hipLaunchKernelGGL(mark_band_kernel<false>, grid, dim3(kBandWaves * 64), lds, stream, routes, lens, S_q, S_k, Lw, bq, bk, bkm,
                         n_rows, words, qw, bitmap);
  } else {
    int rc = launch_fill_i32(reinterpret_cast<int32_t*>(bitmap), static_cast<int64_t>(B) * n_rows * words, 0, stream);
    if (rc) return rc;
    if (qrows > 0) {
      const dim3 grid(static_cast<unsigned>((qrows + kMarkWaves - 1) / kMarkWaves));
      if (vec_routes)
        hipLaunchKernelGGL(mark_kernel<true>, grid, dim3(kMarkWaves * 64), 0, stream, routes, lens, B, S_q, S_k, Lw,
                           bq, bk, bkm, reverse, n_rows, words, bitmap);
      else
        hipLaunchKernelGGL(mark_kernel<false>, grid, dim3(kMarkWaves * 64), 0, stream, routes, lens, B, S_q, S_k, Lw,
                           bq, bk, bkm, reverse, n_rows, words, bitmap);
    }
  }
  if (n_rows > 0 && B > 0) {
    const int vec_in = (words % 4) == 0 && (reinterpret_cast<uintptr_t>(bitmap) & 15) == 0;
    const int vec_out = (width % 4) == 0 && (reinterpret_cast<uintptr_t>(indices) & 15) == 0;
    hipLaunchKernelGGL(emit_kernel, dim3(static_cast<unsigned>(n_rows), static_cast<unsigned>(B)), dim3(256), 0,
                       stream, bitmap, n_rows, words, counts, indices, width, vec_in, vec_out);
  }
  return 0;
}

// Full/partial split of block lists ([FA4] _split_forward_full_blocks,
// _split_backward_full_blocks, _BackwardBlockPartition).  One workgroup per
// list row, its entries in chunks of 256.  Entry o of row r is the block
// (i, j) = (r, o) for forward lists, (o, r) for reverse lists; it is full
// when every query t of tile i routes to every key of tile j.  A route is
// ascending and unique, so query t covers tile j exactly when the entry at
// the first position holding a key >= j*bk (binary search) is j*bk and the
// entry ts - 1 later is the tile's last key (ts = keys in the tile).  The
// (entry, query) tests are spread over the threads; a failing one clears the
// entry's LDS flag, and the flags are compacted in list order into the two
// outputs.  Reads the listed entries once and writes each once.
// One-query tiles: each query's route is read once (one wavefront per query,
// 64 consecutive entries per step) and every key tile it holds completely --
// an entry at a tile's first key whose entry ts - 1 later is the tile's last
// key -- sets bit (t, j) of a [B * S_q, ceil(nkt / 32)] word matrix.
__global__ void __launch_bounds__(kMarkWaves * 64)
cover_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ lens, int B, int S_q, int S_k, int Lw,
             int bk, int words, uint32_t* __restrict__ cover) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kMarkWaves + wid;
  if (row >= static_cast<int64_t>(B) * S_q) return;
  const int n = max(0, min(lens[row], Lw));
  const int32_t* r = routes + row * Lw;
  uint32_t* mrow = cover + row * words;
  for (int e = lane; e < n; e += 64) {
    const int id = r[e];
    if (id < 0 || id >= S_k || id % bk != 0) continue;
    const int ts = min(bk, S_k - id);
    const int last = e + ts - 1;
    if (last < n && r[last] == id + ts - 1) {
      const int j = id / bk;
      atomicOr(&mrow[j >> 5], 1u << (j & 31));
    }
  }
}

// cover != nullptr: one-query tiles (bq = 1) with the coverage bits of
// cover_kernel; otherwise each (entry, query) pair searches the route.
__global__ void __launch_bounds__(256)
split_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ lens, int S_q, int S_k, int Lw, int bq,
             int bk, int reverse, int n_rows, const int32_t* __restrict__ counts, const int32_t* __restrict__ indices,
             int width, int32_t* __restrict__ fc, int32_t* __restrict__ fi, int32_t* __restrict__ pc,
             int32_t* __restrict__ pi, const uint32_t* __restrict__ cover, int words) {
  __shared__ int flag[256];
  __shared__ int ent[256];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int b = blockIdx.y, row = blockIdx.x;
  const int64_t lrow = static_cast<int64_t>(b) * n_rows + row;
  const int cnt = min(max(counts[lrow], 0), width);
  const int32_t* in = indices + lrow * width;
  int32_t* fo = fi + lrow * width;
  int32_t* po = pi + lrow * width;
  int nfull = 0;
  for (int e0 = 0; e0 < cnt; e0 += 256) {
    const int ne = min(256, cnt - e0);
    if (tid < ne) {
      const int o = in[e0 + tid];
      const int i = reverse ? o : row, j = reverse ? row : o;
      ent[tid] = o;
      flag[tid] = (o >= 0 && static_cast<int64_t>(i) * bq < S_q && static_cast<int64_t>(j) * bk < S_k) ? 1 : 0;
    }
    __syncthreads();
    const int64_t npairs = static_cast<int64_t>(ne) * bq;
    for (int64_t p = tid; p < npairs; p += 256) {
      const int e = static_cast<int>(p / bq), qi = static_cast<int>(p % bq);
      const int o = ent[e];
      const int i = reverse ? o : row, j = reverse ? row : o;
      if (o < 0) continue;
      const int64_t tt = static_cast<int64_t>(i) * bq + qi;
      const int64_t k0l = static_cast<int64_t>(j) * bk;
      if (tt >= S_q || k0l >= S_k) continue;
      const int t = static_cast<int>(tt), k0 = static_cast<int>(k0l);
      const int ts = min(bk, S_k - k0);
      const int64_t qrow = static_cast<int64_t>(b) * S_q + t;
      if (cover) {
        if (!((cover[qrow * words + (j >> 5)] >> (j & 31)) & 1u)) atomicAnd(&flag[e], 0);
        continue;
      }
      const int n = max(0, min(lens[qrow], Lw));
      const int32_t* r = routes + qrow * Lw;
      int lo = 0, hi = n;
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (r[m] < k0) lo = m + 1; else hi = m;
      }
      const int last = lo + ts - 1;
      const bool cov = last < n && r[lo] == k0 && r[last] == k0 + ts - 1;
      if (!cov) atomicAnd(&flag[e], 0);
    }
    __syncthreads();
    const int f = tid < ne ? flag[tid] : 0;
    int tot;
    const int incl = block_scan256(f, wsum, &tot);
    if (tid < ne) {
      const int before_full = incl - f;
      if (f) fo[nfull + before_full] = ent[tid];
      else po[(e0 - nfull) + (tid - before_full)] = ent[tid];
    }
    nfull += tot;
    __syncthreads();
  }
  // entries past each count are not written (the lists' readers ignore them):
  // a reverse list of one-query tiles is as wide as the sequence, and filling
  // two such outputs would cost more HBM traffic than the split itself
  if (tid == 0) {
    fc[lrow] = nfull;
    pc[lrow] = cnt - nfull;
  }
}

size_t split_cover_bytes(int B, int S_q, int S_k, int bq, int bk) {
  if (bq != 1 || B < 1 || S_q < 1 || S_k < 1 || bk < 1) return 0;
  const size_t nkt = (static_cast<size_t>(S_k) + bk - 1) / bk;
  return static_cast<size_t>(B) * S_q * ((nkt + 31) / 32) * 4;
}

int launch_split_full_blocks(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int Lw, int bq,
                             int bk, int reverse, const int32_t* counts, const int32_t* indices, int width,
                             int32_t* full_counts, int32_t* full_indices, int32_t* part_counts,
                             int32_t* part_indices, uint32_t* cover, hipStream_t stream) {
  const int nqt = (S_q + bq - 1) / bq, nkt = (S_k + bk - 1) / bk;
  const int n_rows = reverse ? nkt : nqt;
  if (n_rows <= 0 || B <= 0) return 0;
  const int words = (nkt + 31) / 32;
  if (cover) {
    const int64_t qrows = static_cast<int64_t>(B) * S_q;
    int rc = launch_fill_i32(reinterpret_cast<int32_t*>(cover), qrows * words, 0, stream);
    if (rc) return rc;
    hipLaunchKernelGGL(cover_kernel, dim3(static_cast<unsigned>((qrows + kMarkWaves - 1) / kMarkWaves)),
                       dim3(kMarkWaves * 64), 0, stream, routes, lens, B, S_q, S_k, Lw, bk, words, cover);
  }
  hipLaunchKernelGGL(split_kernel, dim3(static_cast<unsigned>(n_rows), static_cast<unsigned>(B)), dim3(256), 0, stream,
                     routes, lens, S_q, S_k, Lw, bq, bk, reverse, n_rows, counts, indices, width, full_counts,
                     full_indices, part_counts, part_indices, cover, words);
  return 0;
}

}  // namespace irb
