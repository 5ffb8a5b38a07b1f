// Internal device/host helpers of libirb (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <limits>
#include <type_traits>

#define IRB_DEV __device__ __forceinline__

namespace irb {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;   // MFMA A/B operand
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;    // 16x16 accumulator
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;  // 32x32 accumulator

// ---------------------------------------------------------------- bf16 <-> f32
IRB_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// round-to-nearest-even (the hardware conversion, v_cvt_pk_bf16_f32: one
// instruction, denormals kept, NaN stays a quiet NaN)
IRB_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// high part = f rounded to bf16; low part = bf16 of the remainder.  hi + lo
// carries ~16 significant bits of f, so a bf16 MFMA against both halves
// reproduces an FP32 product to ~2^-17 relative.
IRB_DEV void split_bf16(float f, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(f);
  lo = f32_to_bf16(f - bf16_to_f32(hi));
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2n;

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest
// even; written out so the pair is never split into two conversions).  The
// inputs must not come straight from an MFMA (see max_raw).
IRB_DEV uint32_t pack_bf16x2(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// 8 floats -> MFMA operand
IRB_DEV bf16x8 pack_bf16x8(const float* f) {
  const uint4 u = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                             pack_bf16x2(f[6], f[7]));
  return __builtin_bit_cast(bf16x8, u);
}
// 2^x on the hardware exp unit (results below the normal range flush to 0,
// which is harmless for softmax weights)
IRB_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> IRB_DEV float load_as_f32(const T* p);
template <> IRB_DEV float load_as_f32<float>(const float* p) { return *p; }
template <> IRB_DEV float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// ---------------------------------------------------------------- wave helpers
IRB_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
IRB_DEV int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
IRB_DEV int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
// inclusive prefix sum over the 64 lanes
IRB_DEV int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Inclusive prefix sum over a 256-thread workgroup; *total receives the
// workgroup's sum.  wsum is 4 ints of LDS; every thread must call it (two
// barriers, the second one keeps wsum alive until everyone has read it).
IRB_DEV int block_scan256(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = wsum[w];
    if (w < wid) off += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return incl + off;
}

// Order LDS traffic between the lanes of ONE wavefront (no cross-wave barrier):
// wait until this wave's LDS operations have completed and stop the compiler
// from moving memory accesses across this point.
IRB_DEV void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- LDS data movement
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).  Vector
// memory operations complete in issue order, so this means "everything but
// the last N issued is done".
template <int N>
constexpr int kVmWaitTile() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  return N | (7 << 4) | (15 << 8);
}

// The same, also waiting for lgkmcnt(0): the wait to use before reading (or
// publishing with a barrier) data that direct global-to-LDS loads wrote.
// Measured on MI355X: after a vmcnt-only wait such data was now and then read
// before it had landed in LDS (one 16-key chunk in roughly one latent
// backward call in ten); with lgkmcnt drained as well no case remained, at
// no measurable cost.
template <int N>
constexpr int kDmaWait() {
  return kVmWaitTile<N>() & ~(15 << 8);
}

// Direct 16-byte global-to-LDS load (global_load_lds_dwordx4): lane i writes
// LDS bytes [lds_base + 16 i, + 16) of the wave-uniform lds_base.  Written as
// inline assembly so that the compiler does not wait for these loads before
// every LDS read; the kernel orders them itself with s_waitcnt vmcnt and a
// barrier.
IRB_DEV void lds_dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_base) : "memory", "m0");
}
// Same with a wave-uniform base address in scalar registers plus a per-lane
// 32-bit unsigned byte offset (the global "saddr" form): the base changes per
// tile in scalar registers while the lane offsets stay in place.
IRB_DEV void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}
// 4-byte direct global-to-LDS load (global_load_lds_dword): lane i writes LDS
// bytes [lds_base + 4 i, + 4); inactive lanes write nothing
IRB_DEV void lds_dma4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(lds_base) : "memory", "m0");
}
IRB_DEV uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
// workgroup barrier that only orders: waits happen where the kernel puts them
IRB_DEV void bare_barrier() {
  asm volatile("" : : : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile in LDS whose
// rows span whole 256-byte bank rounds: chunk c of row r sits at position
// c ^ tr_swz<NC>(r) (NC chunks per row).  It depends on r mod 8 only, so a
// read 8 or 16 rows further is the same pattern at a constant offset.  For
// NC = 16 the row's two low bits go to bits 2-3 and bit 2 to bit 0: the four
// rows x four neighbouring chunks of a 32-lane transpose read
// (ds_read_b64_tr_b16) fall on distinct banks, and 16 consecutive rows read
// at one chunk on pairs of banks.  NC = 8 (128-byte rows): c ^ 2r.
template <int NC>
IRB_DEV int tr_swz(int r) {
  if constexpr (NC >= 16) return ((r & 3) << 2) | ((r >> 2) & 1);
  else return (2 * r) & 7;
}

// LDS transpose read (ds_read_b64_tr_b16): inside each 16-lane row of the
// wavefront, lane 4 a + b receives element b of the 8-byte words that lanes
// a, 4 + a, 8 + a and 12 + a address, in that order.  So if lane s of a row
// addresses row (r0 + s / 4), columns c0 + 4 (s % 4) .. + 3 of a row-major
// bf16 matrix, lane s receives column c0 + s of rows r0 .. r0 + 3: four
// consecutive k of an MFMA A operand whose m is the column.
IRB_DEV v4s lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
}

// Reductions over the four 16-lane rows of a wavefront (lanes l, l^16, l^32,
// l^48) on the VALU: with both operands equal, v_permlane16_swap /
// v_permlane32_swap return {x[l], x[l^16]} / {x[l], x[l^32]} in some order,
// so combining the pair gives the butterfly step without an LDS round trip.
// v_max_f32 without the quieting of its inputs that fmaxf adds for values the
// compiler cannot prove canonical (lane-permute results); NaN inputs are not
// expected here.  Like every inline-assembly helper in this file it must not
// read an MFMA accumulator directly: the compiler does not insert the wait
// states between an MFMA and an inline-assembly reader of its result.
IRB_DEV float max_raw(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
IRB_DEV float max3_raw(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
IRB_DEV float row4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
IRB_DEV float row4_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum of lanes l and l^16 only
IRB_DEV float row_pair_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// ---------------------------------------------------------------- layout
struct Layout {
  int B, S;
  const int32_t* cu_seqlens;   // packed (B == 1) or nullptr
  int num_docs;
  const int32_t* row_lens;     // right-padded rows or nullptr
};

struct Doc {
  int start;   // first token of the document
  int end;     // one past its last token
  int index;   // document index (packed) or 0
  bool valid;  // false for padding tokens
};

IRB_DEV Doc doc_of(const Layout& L, int b, int t) {
  Doc d;
  if (L.cu_seqlens) {
    const int last = L.cu_seqlens[L.num_docs];
    if (t >= last) { d.start = last; d.end = last; d.index = L.num_docs; d.valid = false; return d; }
    int lo = 0, hi = L.num_docs - 1;       // largest i with cu[i] <= t
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (L.cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
    }
    d.start = L.cu_seqlens[lo]; d.end = L.cu_seqlens[lo + 1]; d.index = lo; d.valid = true;
    return d;
  }
  const int n = L.row_lens ? L.row_lens[b] : L.S;
  d.start = 0; d.end = n; d.index = 0; d.valid = t < n;
  return d;
}

// first global block ID of the query's document
IRB_DEV int block_base(const Layout& L, const int32_t* cu_blocks, const Doc& d) {
  return (L.cu_seqlens && cu_blocks) ? cu_blocks[d.index] : 0;
}

// work item -> (b, t, KV head) of the per-query gather kernels: heads
// fastest, or head-major (all queries of a head, then the next head)
struct QItem { int b, t, kvh; };
IRB_DEV QItem decode_qitem(int item, int B, int S_q, int Hkv, int head_major) {
  if (head_major) return QItem{(item / S_q) % B, item % S_q, item / (B * S_q)};
  return QItem{item / (Hkv * S_q), (item / Hkv) % S_q, item % Hkv};
}

// order-preserving uint32 key of a float: larger float -> larger key;
// -0.0 folds onto +0.0; NaN maps below -inf.
IRB_DEV uint32_t score_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace irb
