// Region membership bitmaps of id rows.
//
// CSA page (nemo_automodel...step5.sparse), pack_region_bitmap: each row of
// sorted int32 region ids becomes ceil(regions / 32) membership words (bit
// r % 32 of word r / 32 set when region r occurs in the row), packed directly
// without an int64 scatter workspace; ids at or above `regions` are padding
// and repeats are allowed.  Negative ids are padding here as well (the route
// lists of this library pad with -1), and the rows need not be sorted.
//
// One wavefront per row: the row's words live in the wave's LDS slice; a
// lane takes 8 consecutive ids of each 512-id chunk (16-byte loads when the
// rows are 16-byte aligned), ORs the bits of ids that share a word in
// registers and sets each run's word with one LDS atomic, so sorted rows
// (consecutive ids in one or two words) need few atomics.  The words are
// then written out in one coalesced pass (zeros included), so no output
// clearing pass is needed.
#include "irb_internal.hpp"

namespace irb {

constexpr int kBmWaves = 4;
constexpr int kBmChunks = 4;   // 512-id chunks whose loads are issued together (region bitmaps)
constexpr int kRbChunks = 5;   // the same for route rows (2560 entries: one round for routes of that width)

IRB_DEV void or_run8(uint32_t* bm, const int (&id)[8], int keys) {
  uint32_t acc = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool ok = id[j] >= 0 && id[j] < keys;
    acc |= ok ? 1u << (id[j] & 31) : 0u;
    const int wd = ok ? id[j] >> 5 : -1;
    const int nx = (j < 7 && id[j + 1] >= 0 && id[j + 1] < keys) ? id[j + 1] >> 5 : -2;
    if (wd >= 0 && nx != wd) {
      atomicOr(&bm[wd], acc);
      acc = 0u;
    }
  }
}

__global__ void __launch_bounds__(kBmWaves * 64)
bitmap_kernel(const int32_t* __restrict__ ids, int64_t rows, int slots, int regions, int words, int vec,
              uint32_t* __restrict__ out) {
  extern __shared__ uint32_t bm_all[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kBmWaves + wid;
  if (row >= rows) return;                       // whole wavefront; no workgroup barrier below
  uint32_t* bm = bm_all + wid * words;
  for (int w = lane; w < words; w += 64) bm[w] = 0u;
  const int32_t* r = ids + row * slots;
  wave_lds_sync();
  for (int c0 = 0; c0 < slots; c0 += 512 * kBmChunks) {
    int id[kBmChunks][8];
#pragma unroll
    for (int u = 0; u < kBmChunks; ++u) {
      const int e0 = c0 + 512 * u + 8 * lane;
      if (vec && e0 + 8 <= slots) {
        const int4 a = *reinterpret_cast<const int4*>(r + e0);
        const int4 b = *reinterpret_cast<const int4*>(r + e0 + 4);
        id[u][0] = a.x; id[u][1] = a.y; id[u][2] = a.z; id[u][3] = a.w;
        id[u][4] = b.x; id[u][5] = b.y; id[u][6] = b.z; id[u][7] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) id[u][j] = e0 + j < slots ? r[e0 + j] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kBmChunks; ++u) or_run8(bm, id[u], regions);
  }
  wave_lds_sync();
  uint32_t* o = out + row * words;
  for (int w = lane; w < words; w += 64) o[w] = bm[w];
}

// Key-membership words of ascending route rows with their lengths (the
// forward's query-tile masks): only the first lens[row] entries count.  A
// lane takes 8 consecutive entries of each 512-entry chunk; entries of one
// word are ORed together in registers and the word takes one LDS atomic per
// run, so the long runs of consecutive keys (selected blocks, windows) do not
// serialise on one word.  Rows whose entries are 16-byte aligned (vec) are
// read as int4 pairs, and the loads of up to kRbChunks chunks are issued
// before any of their entries is used.
__global__ void __launch_bounds__(kBmWaves * 64)
route_bits_kernel(const int32_t* __restrict__ routes, const int32_t* __restrict__ lens, int64_t rows, int L,
                  int keys, int words, int vec, uint32_t* __restrict__ out) {
  extern __shared__ uint32_t rb_all[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kBmWaves + wid;
  if (row >= rows) return;                       // whole wavefront; no workgroup barrier below
  uint32_t* bm = rb_all + wid * words;
  for (int w = lane; w < words; w += 64) bm[w] = 0u;
  const int32_t* r = routes + row * L;
  const int n = max(0, min(lens[row], L));
  wave_lds_sync();
  for (int c0 = 0; c0 < n; c0 += 512 * kRbChunks) {
    int id[kRbChunks][8];
#pragma unroll
    for (int u = 0; u < kRbChunks; ++u) {
      const int e0 = c0 + 512 * u + 8 * lane;
      if (vec && e0 + 8 <= L) {
        // the row holds L entries: reading past n stays inside it
        const int4 a = *reinterpret_cast<const int4*>(r + e0);
        const int4 b = *reinterpret_cast<const int4*>(r + e0 + 4);
        const int v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) id[u][j] = e0 + j < n ? v[j] : -1;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) id[u][j] = e0 + j < n ? r[e0 + j] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kRbChunks; ++u) or_run8(bm, id[u], keys);
  }
  wave_lds_sync();
  uint32_t* o = out + row * words;
  for (int w = lane; w < words; w += 64) o[w] = bm[w];
}

int launch_route_bits(const int32_t* routes, const int32_t* lens, int64_t rows, int L, int keys, uint32_t* bits,
                      hipStream_t stream) {
  if (rows == 0) return 0;
  const int words = (keys + 31) / 32;
  const size_t lds = static_cast<size_t>(kBmWaves) * words * sizeof(uint32_t);
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(route_bits_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
  }
  const int vec = (L % 4 == 0 && (reinterpret_cast<uintptr_t>(routes) & 15) == 0) ? 1 : 0;
  hipLaunchKernelGGL(route_bits_kernel, dim3(static_cast<unsigned>((rows + kBmWaves - 1) / kBmWaves)),
                     dim3(kBmWaves * 64), lds, stream, routes, lens, rows, L, keys, words, vec, bits);
  return 0;
}

int launch_bitmap(const int32_t* ids, int64_t rows, int slots, int regions, int32_t* bitmap, hipStream_t stream) {
  if (rows == 0) return 0;
  const int words = (regions + 31) / 32;
  const size_t lds = static_cast<size_t>(kBmWaves) * words * sizeof(uint32_t);
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bitmap_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
  }
  const int vec = (slots % 4 == 0 && (reinterpret_cast<uintptr_t>(ids) & 15) == 0) ? 1 : 0;
  hipLaunchKernelGGL(bitmap_kernel, dim3(static_cast<unsigned>((rows + kBmWaves - 1) / kBmWaves)),
                     dim3(kBmWaves * 64), lds, stream, ids, rows, slots, regions, words, vec,
                     reinterpret_cast<uint32_t*>(bitmap));
  return 0;
}

}  // namespace irb
