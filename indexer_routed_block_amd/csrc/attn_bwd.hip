// a7: sparse GQA attention backward.
//
// Gradients of the routed attention of the QSA page (nemo_automodel...
// qwen3_8_flash_next.qsa, gathered_qsa_gqa_attention: differentiable, indexer
// frozen) for q, k, v; the key side runs over reverse key-to-query lists as
// in the FA4 page (step5.fa4, _selected_block_lists with reverse=True,
// _BackwardBlockPartition).  Latent shared KV (common.cudnn_sparse_attention):
// the merged gradient dK + [dV, 0] lands in one buffer.
//
// No atomics (deterministic).  Launches:
//  delta Delta[b,h,t] = rowsum(dO * o) from the forward kernel run again with
//        o kept in FP32 (the stored bf16 output would put its rounding into
//        every dS of the row, and dK sums those coherently).
//  dq    per (query, KV head): like the forward, S^T = K Q^T and
//        dP^T = V dO^T on gathered rows, dS^T = P^T (dP^T - Delta),
//        dQ^T += K^T dS^T with K^T read transposed from LDS.
//  dK/dV, bf16 with D = Dv in {64, 128} (the GQA configurations):
//   hits  per 16-key tile, the reverse list's queries whose routes hold one of
//         its keys, ascending, each with its 16-bit key mask (a counting pass,
//         a prefix sum, a filling pass), so the MFMA kernel never searches.
//   dkdv  per (16-key tile, KV head), one wavefront: K and V of the tile stay
//         in registers as B operands; 32 (query, head) rows at a time are
//         loaded straight into the A layout for S = Q K^T and dP = dO V^T and
//         copied row-major to a per-wave LDS slab; dV^T += dO^T P and
//         dK^T += Q^T dS then take their A operands from the slab with LDS
//         transpose reads, and P, dS straight from the accumulators as B
//         operands (bf16 high + low halves, so the long key-side sums keep
//         FP32 accuracy).
//  dK/dV otherwise (fp32 inputs, latent 576/512):
//   prep  copies of q and dO with the heads of a KV group innermost
//         ([b, t, kvh, dim, Gp]) so that the key-side MFMAs can read
//         (rows x dims)^T operands with 8/16-byte loads.
//   dkdv  per (16-key tile, KV head), one wavefront: walks the reverse list,
//         finds each listed query's keys inside the tile by binary search in
//         its ascending route, packs hitting queries 32 (query, head) rows at
//         a time and accumulates dV^T += dO^T P and dK^T += q^T dS in
//         registers.
#include <algorithm>

#include "irb_internal.hpp"

namespace irb {

constexpr float kLog2eB = 1.4426950408889634f;

IRB_DEV void bld8(const uint16_t* p, bf16x8& hi, bf16x8& lo) {
  hi = *reinterpret_cast<const bf16x8*>(p);
  (void)lo;
}
IRB_DEV void bld8(const float* p, bf16x8& hi, bf16x8& lo) {
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
// 4 consecutive elements into operand slots [o, o+4)
IRB_DEV void bld4(const uint16_t* p, bf16x8& hi, bf16x8& lo, int o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  hi[o + 0] = static_cast<short>(u.x & 0xffffu);
  hi[o + 1] = static_cast<short>(u.x >> 16);
  hi[o + 2] = static_cast<short>(u.y & 0xffffu);
  hi[o + 3] = static_cast<short>(u.y >> 16);
  (void)lo;
}
IRB_DEV void bld4(const float* p, bf16x8& hi, bf16x8& lo, int o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float f[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t h, l;
    split_bf16(f[e], h, l);
    hi[o + e] = static_cast<short>(h);
    lo[o + e] = static_cast<short>(l);
  }
}
IRB_DEV void bzero8(bf16x8& x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0;
}
IRB_DEV void bput(bf16x8& hi, bf16x8& lo, int e, uint16_t v) { hi[e] = static_cast<short>(v); (void)lo; }
IRB_DEV void bput(bf16x8& hi, bf16x8& lo, int e, float v) {
  uint16_t h, l;
  split_bf16(v, h, l);
  hi[e] = static_cast<short>(h);
  lo[e] = static_cast<short>(l);
}
IRB_DEV void bput_f(bf16x8& hi, bf16x8& lo, int e, float v, bool split) {
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
IRB_DEV f32x4 bmma(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  if (kSplit) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  }
  return acc;
}
// acc += a * (b_hi + b_lo), plus a_lo * b_hi when a is itself split (FP32 inputs)
template <bool kSplitA>
IRB_DEV f32x4 bmma_split_b(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  if (kSplitA) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  return acc;
}
IRB_DEV void bstore4(uint16_t* p, const float* v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
IRB_DEV void bstore4(float* p, const float* v) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }
IRB_DEV void bcopy16(void* dst, const void* src, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *reinterpret_cast<const uint4*>(src);
  *reinterpret_cast<uint4*>(dst) = v;
}

// heads of a KV group padded so that 4 consecutive rows are 4 heads of one
// query and 32 rows hold whole queries (or a query holds whole 32-row blocks)
static int padded_group(int G) {
  if (G <= 4) return 4;
  if (G <= 8) return 8;
  if (G <= 16) return 16;
  if (G <= 32) return 32;
  return (G + 31) / 32 * 32;
}

// bf16 GQA shapes and the bf16 latent shape with whole 32-head batches take
// the hit-list path; the rest the transposed-copy path
static bool uses_hits(int dtype, int Dqk, int Dv, int G) {
  if (dtype != IRB_BF16) return false;
  if (Dqk == Dv && (Dqk == 64 || Dqk == 128)) return true;
  return Dqk == 576 && Dv == 512 && G % 32 == 0;
}

struct BwdWs {
  float* delta;       // [B, Hq, S_q]
  void* qt;           // transposed path: [B, S_q, Hkv, Dqk, Gp]
  void* dot;          //                  [B, S_q, Hkv, Dv, Gp]
  int64_t* hit_off;   // hit path: [RG * B * nkt + 1] counts, then exclusive offsets
  int32_t* hit_t;     //           [cap] query of each hit
  uint32_t* hit_m;    //           [cap] its 16-bit key mask
  int64_t cap;        // every (group, key tile, query) with a routed key: <= RG * B * S_q * min(L, nkt)
  // union lists of 64-key groups (bf16 GQA): counts then offsets, queries, four 16-bit masks each
  int64_t* off64;     // [RG * B * ngrp + 1]
  int32_t* t64;       // [cap64]
  uint16_t* m64;      // [cap64][4]
  int64_t cap64;      // <= RG * B * S_q * min(L, ngrp)
  int32_t* ord;       // [B * ngrp * Hkv] dispatch order of the key-side workgroups
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t hit_capacity(int B, int S_q, int S_k, int L, int RG) {
  const int64_t nkt = (static_cast<int64_t>(S_k) + 15) / 16;
  return static_cast<int64_t>(RG) * B * S_q * std::min<int64_t>(L, nkt);
}

// the key side's union lists of 64-key groups: bf16 GQA shapes whose query
// bitmap (S_q bits plus a count per word) fits 64 KiB of LDS
static bool uses_union(int dtype, int Dqk, int Dv, int S_q) {
  static const bool on = [] {
    const char* e = getenv("IRB_KEY_UNION");
    return !(e && e[0] == '0');
  }();
  return on && dtype == IRB_BF16 && Dqk == Dv && (Dqk == 64 || Dqk == 128) &&
         (static_cast<int64_t>(S_q) + 31) / 32 * 8 <= 65536;
}
// least overlap (per mille: sum of a 64-key group's four tile-list counts
// over its union count) for the shared-batch key side, 1.5 (measured best of
// 1.0-3: lower sends groups whose tiles share few queries through batches
// that reach one tile each); IRB_KEY_UNION_MIN_OVERLAP overrides it
static int key_overlap_milli() {
  static const int v = [] {
    const char* e = getenv("IRB_KEY_UNION_MIN_OVERLAP");
    return e ? static_cast<int>(atof(e) * 1000.0) : 1500;
  }();
  return v;
}
static int64_t union_capacity(int B, int S_q, int S_k, int L, int RG) {
  const int64_t ngrp = (static_cast<int64_t>(S_k) + 63) / 64;
  return static_cast<int64_t>(RG) * B * S_q * std::min<int64_t>(L, ngrp);
}

size_t attn_bwd_workspace_bytes(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv, int dtype,
                                int RG) {
  const int G = Hq / (Hkv > 0 ? Hkv : 1);
  const size_t Gp = static_cast<size_t>(padded_group(G));
  const size_t rows = static_cast<size_t>(B) * S_q;
  size_t n = align256(rows * Hq * 4);
  if (uses_hits(dtype, Dqk, Dv, G)) {
    const size_t nkt = (static_cast<size_t>(S_k) + 15) / 16;
    const size_t cap = static_cast<size_t>(hit_capacity(B, S_q, S_k, L, RG));
    n += align256((static_cast<size_t>(RG) * B * nkt + 1) * 8) + 2 * align256(cap * 4);
    if (G <= 32 && uses_union(dtype, Dqk, Dv, S_q)) {
      const size_t ngrp = (static_cast<size_t>(S_k) + 63) / 64;
      const size_t cap64 = static_cast<size_t>(union_capacity(B, S_q, S_k, L, RG));
      n += align256((static_cast<size_t>(RG) * B * ngrp + 1) * 8) + align256(cap64 * 4) + align256(cap64 * 8) +
           align256(static_cast<size_t>(B) * ngrp * Hkv * 4);
    }
    // 64 heads over shared latent rows: the query-major path (used when v aliases k)
    if (dtype == IRB_BF16 && Dqk == 576 && Dv == 512 && G == 64)
      n = std::max(n, latent_bwd_workspace_bytes(B, S_q, S_k, L, Hq, Hkv));
  } else {
    const size_t esz = dtype == IRB_BF16 ? 2 : 4;
    n += align256(rows * Hkv * Dqk * Gp * esz) + align256(rows * Hkv * Dv * Gp * esz);
  }
  return n;
}

// whether the backward reads Delta off the forward's FP32 output when given
// one: where a pass would otherwise form it (the query-tile dQ, a forward in
// Delta mode, the latent path), not where the per-query dQ pass forms it
// anyway (row strides as in contiguous q / k / v assumed)
bool attn_bwd_reads_out32(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv, int dtype, int RG) {
  if (B < 1 || S_q < 1 || S_k < 1 || L < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  if (dtype == IRB_BF16 && Dqk == 576 && Dv == 512 && G == 64) return true;
  const bool fused = dtype == IRB_BF16 && Dqk <= 128 && G <= 16;
  if (!fused) return true;
  if (!(Dqk == Dv && (Dqk == 64 || Dqk == 128)) || !(G == 4 || G == 8 || G == 16)) return false;
  AttnArgs a{};
  a.B = B; a.S_q = S_q; a.S_k = S_k; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.Dqk = Dqk; a.Dv = Dv;
  a.dtype = dtype; a.RG = RG;
  const size_t qb = attn_fwd_qbits_bytes(a);
  const size_t room = 2 * align256(static_cast<size_t>(hit_capacity(B, S_q, S_k, L, RG)) * 4);
  return tile_thr_milli() <= 1000 && qb > 0 && qb <= room;
}

static BwdWs carve(void* ws, int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv, int dtype, int RG) {
  const int G = Hq / Hkv;
  const size_t Gp = static_cast<size_t>(padded_group(G));
  const size_t rows = static_cast<size_t>(B) * S_q;
  char* p = static_cast<char*>(ws);
  BwdWs w{};
  w.delta = reinterpret_cast<float*>(p);
  p += align256(rows * Hq * 4);
  if (uses_hits(dtype, Dqk, Dv, G)) {
    const size_t nkt = (static_cast<size_t>(S_k) + 15) / 16;
    w.cap = hit_capacity(B, S_q, S_k, L, RG);
    w.hit_off = reinterpret_cast<int64_t*>(p);
    p += align256((static_cast<size_t>(RG) * B * nkt + 1) * 8);
    w.hit_t = reinterpret_cast<int32_t*>(p);
    p += align256(static_cast<size_t>(w.cap) * 4);
    w.hit_m = reinterpret_cast<uint32_t*>(p);
    p += align256(static_cast<size_t>(w.cap) * 4);
    if (G <= 32 && uses_union(dtype, Dqk, Dv, S_q)) {
      const size_t ngrp = (static_cast<size_t>(S_k) + 63) / 64;
      w.cap64 = union_capacity(B, S_q, S_k, L, RG);
      w.off64 = reinterpret_cast<int64_t*>(p);
      p += align256((static_cast<size_t>(RG) * B * ngrp + 1) * 8);
      w.t64 = reinterpret_cast<int32_t*>(p);
      p += align256(static_cast<size_t>(w.cap64) * 4);
      w.m64 = reinterpret_cast<uint16_t*>(p);
      p += align256(static_cast<size_t>(w.cap64) * 8);
      w.ord = reinterpret_cast<int32_t*>(p);
    }
  } else {
    const size_t esz = dtype == IRB_BF16 ? 2 : 4;
    w.qt = p;
    p += align256(rows * Hkv * Dqk * Gp * esz);
    w.dot = p;
  }
  return w;
}

// ---------------------------------------------------------------- prep
template <typename T>
__global__ void __launch_bounds__(256)
bwd_prep_kernel(AttnArgs a, const T* __restrict__ dout, T* __restrict__ qt, T* __restrict__ dot, int G, int Gp) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;             // b * S_q + t
  const int b = static_cast<int>(row / a.S_q), t = static_cast<int>(row % a.S_q);
  // transposed copies: [kvh][dim][hp]
  const T* qrow = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t;
  T* qdst = qt + row * a.Hkv * a.Dqk * Gp;
  for (int i = tid; i < a.Hkv * a.Dqk * Gp; i += 256) {
    const int hp = i % Gp, d = (i / Gp) % a.Dqk, g = i / (Gp * a.Dqk);
    qdst[i] = (hp < G) ? qrow[static_cast<int64_t>(g * G + hp) * a.sq_h + d] : T(0);
  }
  const T* drow = dout + row * a.Hq * a.Dv;
  T* ddst = dot + row * a.Hkv * a.Dv * Gp;
  for (int i = tid; i < a.Hkv * a.Dv * Gp; i += 256) {
    const int hp = i % Gp, d = (i / Gp) % a.Dv, g = i / (Gp * a.Dv);
    ddst[i] = (hp < G) ? drow[static_cast<int64_t>(g * G + hp) * a.Dv + d] : T(0);
  }
}

// ---------------------------------------------------------------- delta from the FP32 output
// Delta[b, h, t] = sum_d dO[b, t, h, d] o[b, t, h, d] with the forward's FP32
// o: 16 lanes per (row, head), four elements per lane and step, summed
// across the 16 lanes
template <typename T>
__global__ void __launch_bounds__(256)
delta_from_o_kernel(const T* __restrict__ dout, const float* __restrict__ o32, float* __restrict__ delta, int B,
                    int S_q, int Hq, int Dv) {
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4;   // (row, head)
  const int l = threadIdx.x & 15;
  const int64_t n = static_cast<int64_t>(B) * S_q * Hq;
  const bool ok = g < n;
  float part = 0.f;
  if (ok) {
    const T* dp = dout + g * Dv;
    const float* op = o32 + g * Dv;
    for (int d = 4 * l; d < Dv; d += 64) {
      const float4 o = *reinterpret_cast<const float4*>(op + d);
      part += load_as_f32(dp + d) * o.x + load_as_f32(dp + d + 1) * o.y + load_as_f32(dp + d + 2) * o.z +
              load_as_f32(dp + d + 3) * o.w;
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 16);
  if (ok && l == 0) {
    const int h = static_cast<int>(g % Hq);
    const int64_t bt = g / Hq;
    const int b = static_cast<int>(bt / S_q), t = static_cast<int>(bt % S_q);
    delta[(static_cast<int64_t>(b) * Hq + h) * S_q + t] = part;
  }
}

int launch_delta_from_o(const AttnArgs& a, const void* dout, const float* o32, float* delta, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(a.B) * a.S_q * a.Hq;
  if (groups == 0) return 0;
  const dim3 grid(static_cast<unsigned>((groups * 16 + 255) / 256));
  if (a.dtype == IRB_BF16)
    hipLaunchKernelGGL(delta_from_o_kernel<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(dout),
                       o32, delta, a.B, a.S_q, a.Hq, a.Dv);
  else
    hipLaunchKernelGGL(delta_from_o_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(dout), o32,
                       delta, a.B, a.S_q, a.Hq, a.Dv);
  return 0;
}

// ---------------------------------------------------------------- dq
// bf16, one wavefront per (batch, query, KV head) with G <= 16 heads as the
// MFMA columns; this pass also forms the row statistic Delta.  Per 32-key
// chunk: S^T = K Q^T and dP^T = V dO^T with the gathered K and V rows as A
// operands, P = exp(S - lse), and, with K^T from the wave's LDS slab
// (row-major copy of the chunk's K rows) by transpose reads,
//   A^T += K^T (P dP)^T,   B^T += K^T P^T,   Delta += sum_k P dP,
// so that dQ = scale (A - Delta B) = scale sum_k P (dP - Delta) k without a
// separate pass for Delta.  P dP and P enter as bf16 high + low parts, so A
// and B carry ~16 significant bits and their difference stays accurate.
// Delta = sum_k P dP equals rowsum(dO o) for the FP32 o.  The next chunk's K
// and V rows load while the current chunk's softmax and dQ work runs.
template <int D, int DV>
IRB_DEV void dq_item_gather(const AttnArgs& a, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                            float* __restrict__ delta, uint16_t* __restrict__ dq, int G, int b, int t, int kvh,
                            uint16_t* kl) {
  using T = uint16_t;
  constexpr int KS = D / 32, VS = DV / 32, NDQ = D / 16;
  constexpr int LDK = D + 8;
  const int lane = threadIdx.x & 63;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int h0 = kvh * G;
  const int nh = min(16, G);
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;
  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  const bool hok = l16 < nh;
  const int hh = h0 + (hok ? l16 : 0);
  bf16x8 qh[KS], dh[VS];
  {
    const T* qp = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qh[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
      if (!hok) bzero8(qh[s]);
    }
    const T* dp = dout + (row * a.Hq + hh) * DV + 8 * g16;
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      dh[s] = *reinterpret_cast<const bf16x8*>(dp + 32 * s);
      if (!hok) bzero8(dh[s]);
    }
  }
  const float lse2 = hok ? lse[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] * kLog2eB : 0.f;
  const float sc2 = a.scale * kLog2eB;
  f32x4 acc[NDQ], accb[NDQ];
#pragma unroll
  for (int i = 0; i < NDQ; ++i) { acc[i] = f32x4{0.f, 0.f, 0.f, 0.f}; accb[i] = acc[i]; }
  float dsum = 0.f;
  const int vk0 = 4 * g16 + (l16 >> 2);   // K^T transpose reads: first key row

  struct Pre { bf16x8 k[2][KS], v[2][VS]; };
  auto load = [&](int e0, Pre& r) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int e = e0 + 16 * ti + l16;
      const int id = e < n ? route[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      const T* kr = kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t + 8 * g16;
      const T* vr = vbase + static_cast<int64_t>(ok ? id : 0) * a.sv_t + 8 * g16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        r.k[ti][s] = *reinterpret_cast<const bf16x8*>(kr + 32 * s);
        if (!ok) bzero8(r.k[ti][s]);
      }
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        r.v[ti][s] = *reinterpret_cast<const bf16x8*>(vr + 32 * s);
        if (!ok) bzero8(r.v[ti][s]);
      }
    }
  };
  auto step = [&](int e0, Pre& pf) __attribute__((always_inline)) {
    // row-major copy of the chunk's K rows for the transposed operand
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<bf16x8*>(kl + (16 * ti + l16) * LDK + 8 * g16 + 32 * s) = pf.k[ti][s];
    f32x4 st[2], dpt[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      st[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpt[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) st[ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf.k[ti][s], qh[s], st[ti], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < VS; ++s) dpt[ti] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf.v[ti][s], dh[s], dpt[ti], 0, 0, 0);
    }
    wave_lds_sync();
    if (e0 + 32 < n) load(e0 + 32, pf);
    // P and P dP at keys 16 ti + 4 g16 + i, column = head l16
    bf16x8 ph, pl, qh2, ql2;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * ti + 4 * g16 + i;
        const float p = (e < n && hok) ? exp2f(st[ti][i] * sc2 - lse2) : 0.f;
        const float pd = p * dpt[ti][i];
        dsum += pd;
        bput_f(ph, pl, 4 * ti + i, p, true);
        bput_f(qh2, ql2, 4 * ti + i, pd, true);
      }
    // A^T += K^T (P dP)^T and B^T += K^T P^T; k-slot j is key 4 g16 + j
    // (j < 4) or 16 + 4 g16 + (j - 4)
#pragma unroll
    for (int dt = 0; dt < NDQ; ++dt) {
      const T* w = kl + vk0 * LDK + 16 * dt + 4 * (l16 & 3);
      const v4s x0 = lds_read_tr(w), x1 = lds_read_tr(w + 16 * LDK);
      const bf16x8 xa = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, qh2, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ql2, acc[dt], 0, 0, 0);
      accb[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ph, accb[dt], 0, 0, 0);
      accb[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, pl, accb[dt], 0, 0, 0);
    }
    wave_lds_sync();   // the slab is rewritten by the next chunk
  };
  if (n > 0) {
    Pre pf;
    load(0, pf);
    for (int e0 = 0; e0 < n; e0 += 32) step(e0, pf);
  }
  const float dlt = row4_sum(dsum);
  if (hok) {
    if (g16 == 0) delta[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] = dlt;
    T* op = dq + (row * a.Hq + h0 + l16) * D + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDQ; ++dt) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (acc[dt][i] - dlt * accb[dt][i]) * a.scale;
      bstore4(op + dt * 16, v);
    }
  }
}

// whether the query side forms Delta itself (dq_item_gather)
template <typename T, int D>
constexpr bool dq_fuses_delta() { return sizeof(T) == 2 && D <= 128; }

template <typename T, int D, int DV, bool kShared>
__global__ void __launch_bounds__(256, (!kShared && dq_fuses_delta<T, D>()) ? 2 : 1)
bwd_dq_kernel(AttnArgs a, const T* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ delta,
              T* __restrict__ dq, int G, int n_items, int latent, int head_major, int tile_bq, int thr_milli) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int KS = D / 32, VS = DV / 32, NDQ = D / 16;
  constexpr int PAD = sizeof(T) == 2 ? 8 : 4;
  constexpr int LDK = D + PAD, LDV = DV + PAD;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  int item, slice;
  if (kShared) { item = blockIdx.x; slice = wid; }
  else { item = blockIdx.x * 4 + wid; slice = 0; if (item >= n_items) return; }
  const QItem qi = decode_qitem(item, a.B, a.S_q, a.Hkv, kShared ? 0 : head_major);
  const int kvh = qi.kvh, t = qi.t, b = qi.b;
  if constexpr (!kShared && dq_fuses_delta<T, D>()) {
    // the query-tile kernel's tiles (same test) are not this launch's
    if (tile_bq > 0 && tile_stats_wave(a, b, kvh, (t / tile_bq) * tile_bq, tile_bq, thr_milli).dense) return;
    dq_item_gather<D, DV>(a, dout, lse, delta, dq, G, b, t, kvh,
                          reinterpret_cast<uint16_t*>(smem) + wid * 32 * (D + 8));
    return;
  }
  const int h0 = kvh * G + 16 * slice;
  const int nh = min(16, G - 16 * slice);
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;
  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  const bool hok = l16 < nh;
  const int hh = h0 + (hok ? l16 : 0);

  bf16x8 qh[KS], ql[KS], dh[VS], dl[VS];
  {
    const T* qp = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) { bld8(qp + 32 * s, qh[s], ql[s]); if (!hok) { bzero8(qh[s]); bzero8(ql[s]); } }
    const T* dp = dout + (row * a.Hq + hh) * DV + 8 * g16;
#pragma unroll
    for (int s = 0; s < VS; ++s) { bld8(dp + 32 * s, dh[s], dl[s]); if (!hok) { bzero8(dh[s]); bzero8(dl[s]); } }
  }
  const float lse2 = hok ? lse[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] * kLog2eB : 0.f;
  const float dlt = hok ? delta[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] : 0.f;
  const float sc2 = a.scale * kLog2eB;
  f32x4 acc[NDQ];
#pragma unroll
  for (int i = 0; i < NDQ; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  T* kl = kShared ? reinterpret_cast<T*>(smem) : reinterpret_cast<T*>(smem) + wid * 32 * LDK;
  T* vl = kl + 32 * LDK;   // shared, non-latent only
  for (int e0 = 0; e0 < n; e0 += 32) {
    if (kShared) {
      __syncthreads();
      constexpr int K16 = D * static_cast<int>(sizeof(T)) / 16;
      for (int i = threadIdx.x; i < 32 * K16; i += blockDim.x) {
        const int kk = i / K16, c16 = i % K16;
        const int e = e0 + kk;
        const int id = e < n ? route[e] : -1;
        const bool ok = id >= 0 && id < a.S_k;
        bcopy16(reinterpret_cast<char*>(kl + kk * LDK) + 16 * c16,
                reinterpret_cast<const char*>(kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t) + 16 * c16, ok);
      }
      if (!latent) {
        constexpr int V16 = DV * static_cast<int>(sizeof(T)) / 16;
        for (int i = threadIdx.x; i < 32 * V16; i += blockDim.x) {
          const int kk = i / V16, c16 = i % V16;
          const int e = e0 + kk;
          const int id = e < n ? route[e] : -1;
          const bool ok = id >= 0 && id < a.S_k;
          bcopy16(reinterpret_cast<char*>(vl + kk * LDV) + 16 * c16,
                  reinterpret_cast<const char*>(vbase + static_cast<int64_t>(ok ? id : 0) * a.sv_t) + 16 * c16, ok);
        }
      }
      __syncthreads();
    } else {
      constexpr int K16 = D * static_cast<int>(sizeof(T)) / 16;
      const int kk = lane >> 1, hf = lane & 1;
      const int e = e0 + kk;
      const int id = e < n ? route[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      const char* src = reinterpret_cast<const char*>(kbase + static_cast<int64_t>(ok ? id : 0) * a.sk_t);
      char* dst = reinterpret_cast<char*>(kl + kk * LDK);
      for (int c16 = hf; c16 < K16; c16 += 2) bcopy16(dst + 16 * c16, src + 16 * c16, ok);
      wave_lds_sync();
    }
    f32x4 st[2], dpt[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      st[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpt[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* kr = kl + (16 * ti + l16) * LDK + 8 * g16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 xh, xl;
        bld8(kr + 32 * s, xh, xl);
        st[ti] = bmma<kSplit>(xh, xl, qh[s], ql[s], st[ti]);
      }
      const T* vr;
      bool vok = true;
      if (kShared) {
        vr = (latent ? kl + (16 * ti + l16) * LDK : vl + (16 * ti + l16) * LDV) + 8 * g16;
      } else {
        const int e = e0 + 16 * ti + l16;
        const int id = e < n ? route[e] : -1;
        vok = id >= 0 && id < a.S_k;
        vr = vbase + static_cast<int64_t>(vok ? id : 0) * a.sv_t + 8 * g16;
      }
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        bf16x8 xh, xl;
        bld8(vr + 32 * s, xh, xl);
        if (!vok) { bzero8(xh); bzero8(xl); }
        dpt[ti] = bmma<kSplit>(xh, xl, dh[s], dl[s], dpt[ti]);
      }
    }
    float ds[2][4];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * ti + 4 * g16 + i;
        const float p = (e < n && hok) ? exp2f(st[ti][i] * sc2 - lse2) : 0.f;
        ds[ti][i] = p * (dpt[ti][i] - dlt);
      }
    bf16x8 sh, sl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bput_f(sh, sl, j, ds[0][j], kSplit);
      bput_f(sh, sl, 4 + j, ds[1][j], kSplit);
    }
#pragma unroll
    for (int dt = 0; dt < NDQ; ++dt) {
      bf16x8 xh, xl;
      const T* kc = kl + dt * 16 + l16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = (j < 4) ? 4 * g16 + j : 16 + 4 * g16 + (j - 4);
        bput(xh, xl, j, kc[kk * LDK]);
      }
      acc[dt] = bmma<kSplit>(xh, xl, sh, sl, acc[dt]);
    }
    if (!kShared) {
      wave_lds_sync();
    }
  }
  if (hok) {
    T* op = dq + (row * a.Hq + h0 + l16) * D + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDQ; ++dt) {
      const float v[4] = {acc[dt][0] * a.scale, acc[dt][1] * a.scale, acc[dt][2] * a.scale, acc[dt][3] * a.scale};
      bstore4(op + dt * 16, v);
    }
  }
}

// ---------------------------------------------------------------- dq, query tiles
// XOR swizzle of the dq tile kernel's K and V rows (NC 16-byte chunks per
// row): chunk c of row r at position c ^ dqt_swz<NC>(r).  NC = 16: row bits
// 0, 1 to bits 2, 3 and bits 2, 3 to bits 0, 1 -- a permutation, so the 16
// rows of a 16-lane row read fall on distinct banks, and four consecutive
// rows take distinct bits 2-3, so the 32-lane transpose reads (four rows x
// four neighbouring chunks) do too.  Row r + 8 (r < 8) is row r's pattern
// with bit 1 flipped, row r + 16 the same pattern.  NC = 8: c ^ 2r.
template <int NC>
IRB_DEV int dqt_swz(int r) {
  if constexpr (NC >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (2 * r) & 7;
}


// bf16 GQA with D = Dv in {64, 128} and G in {4, 8, 16}: one workgroup per
// (query tile of 128 / G queries, KV head), organised like the forward's
// query-tile kernel.  The tile's 128 (query, head) pairs are the MFMA columns
// (wave w holds pairs 32 w .. 32 w + 31); the 32-key tiles that any of its
// queries routes to stream through LDS by direct loads (two slots: the next
// tile loads while the current one is used); each query's key-membership
// words (built once per call) mask them.  Two sweeps over those key tiles:
//   1: S^T = K Q^T, dP^T = V dO^T, P = exp(S - lse) on routed keys,
//      Delta += sum_k P dP in FP32;
//   2: S^T, dP^T and P again, dS = P (dP - Delta) in FP32, rounded once to
//      bf16, and dQ^T += K^T dS^T with K^T from LDS transpose reads.  dS is
//      formed before the rounding, so each term carries only its own
//      relative rounding (no cancellation is rounded in).
// dQ = scale (dQ^T)^T; Delta is written for the key side.  With Delta given
// (have_delta: computed from the forward's FP32 output) only sweep 2 runs.  Query tiles whose
// routes cover too little of their key range go per query (dq_item_gather):
// here when gather_rest, else in the per-query launch, which skips this
// kernel's tiles by the same test.
template <int D, int G>
__global__ void __launch_bounds__(256, 2)
bwd_dq_tile_kernel(AttnArgs a, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                   float* __restrict__ delta, uint16_t* __restrict__ dq, int n_qt, int thr_milli,
                   const uint32_t* __restrict__ qbits, int qwords, int gather_rest, int have_delta) {
  using T = uint16_t;
  constexpr int BQ = 128 / G;
  constexpr int KS = D / 16;     // 16-dim k-steps of S^T and dP^T
  constexpr int NDT = D / 32;    // 32-dim row tiles of dQ^T
  constexpr int NC = D / 8;      // 16-byte chunks per K or V row
  // K and V rows of a key tile, row-major (K first), chunk c of row r at slot
  // c ^ dqt_swz(r)
  constexpr int KBYTES = 32 * D * 2;
  constexpr int BUF = 2 * KBYTES;
  constexpr int NI = 32 * NC / 256;        // direct loads per wave per tile side
  constexpr int SLAB = 32 * (D + 8) * 2;   // per-wave LDS of dq_item_gather
  constexpr int RAW = 2 * BUF > 4 * SLAB ? 2 * BUF : 4 * SLAB;
  static_assert(NI >= 1, "tile loads");
  __shared__ __align__(16) char raw[RAW];
  __shared__ uint32_t mask[BQ][kSegTiles + 1];
  __shared__ int tiles[kSegTiles];
  __shared__ int s_ntiles;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  // grid order as the forward's tile kernel: KV heads of one query tile
  // adjacent, query tiles last-first
  const int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  const int qt = n_qt - 1 - (bid / a.Hkv) % n_qt;
  const int b = bid / (a.Hkv * n_qt);
  const int qa = qt * BQ;
  const TileStats ts = tile_stats_wave(a, b, kvh, qa, BQ, thr_milli);
  if (!ts.dense) {
    if (!gather_rest) return;
    T* slab = reinterpret_cast<T*>(raw + wid * SLAB);
    for (int q = wid; q < BQ; q += 4)
      if (qa + q < a.S_q) dq_item_gather<D, D>(a, dout, lse, delta, dq, G, b, qa + q, kvh, slab);
    return;
  }

  const T* kbase = static_cast<const T*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.sv_b + kvh * a.sv_h;
  // this lane's column (query colq of the tile, head colh of the group); MFMA
  // layout (v_mfma_f32_32x32x16_bf16): A lane l = row l % 32, k 8 (l / 32) ..
  // + 8; B lane l = column l % 32, same k; accumulator element i of lane l =
  // row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
  const int col = 32 * wid + l32;
  const int colq = col / G, colh = col % G;
  const int t = qa + colq;
  const bool tok = t < a.S_q;
  const int hh = kvh * G + colh;
  bf16x8 qop[KS], dop[KS];
  {
    const int tt = tok ? t : 0;
    const T* qp = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(tt) * a.sq_t +
                  static_cast<int64_t>(hh) * a.sq_h + 8 * h32;
    const T* dp = dout + ((static_cast<int64_t>(b) * a.S_q + tt) * a.Hq + hh) * D + 8 * h32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
      dop[s] = *reinterpret_cast<const bf16x8*>(dp + 16 * s);
      if (!tok) { bzero8(qop[s]); bzero8(dop[s]); }
    }
  }
  const float lse2 = tok ? lse[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] * kLog2eB : 0.f;
  const float sc2 = a.scale * kLog2eB;

  // tile loader: lane i of wave w's load n fills 16-byte slot (w NI + n) 64 + i
  // of the K (or V) half; the global address is the tile's first row (scalar
  // registers) plus a per-lane 32-bit byte offset fixed for the whole kernel
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int slot = (wv * NI + n) * 64 + lane;
    const int r = slot / NC, sw = (slot % NC) ^ dqt_swz<NC>(r);
    koff[n] = static_cast<uint32_t>(r * a.sk_t + 8 * sw) * 2u;
    voff[n] = static_cast<uint32_t>(r * a.sv_t + 8 * sw) * 2u;
  }
  const uint32_t lds0 = lds_addr(raw);
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    kt = __builtin_amdgcn_readfirstlane(kt);
    buf = __builtin_amdgcn_readfirstlane(buf);
    const int key0 = kt * 32;
    const T* ks = kbase + static_cast<int64_t>(key0) * a.sk_t;
    const T* vs = vbase + static_cast<int64_t>(key0) * a.sv_t;
    const int lim = a.S_k - 1 - key0;
    const uint32_t ld = lds0 + buf * BUF + wv * NI * 1024;
    if (lim >= 31) {
#pragma unroll
      for (int n = 0; n < NI; ++n) lds_dma16_s(ks, koff[n], ld + n * 1024);
#pragma unroll
      for (int n = 0; n < NI; ++n) lds_dma16_s(vs, voff[n], ld + KBYTES + n * 1024);
    } else {
      // the last tile: rows past the last key repeat it (their keys are never routed)
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int slot = (wv * NI + n) * 64 + lane;
        const int r = slot / NC, sw = (slot % NC) ^ dqt_swz<NC>(r);
        const int rr = min(r, lim);
        lds_dma16_s(ks, static_cast<uint32_t>(rr * a.sk_t + 8 * sw) * 2u, ld + n * 1024);
        lds_dma16_s(vs, static_cast<uint32_t>(rr * a.sv_t + 8 * sw) * 2u, ld + KBYTES + n * 1024);
      }
    }
  };
  // per-lane LDS byte offsets inside a slot.  Row reads (A = K or V rows, k =
  // dims): row l32, chunk 2 s + h32.  K^T transpose reads of dim tile dt:
  // lanes of a 16-lane row address keys 4 h32 + (lane % 16) / 4 (+ 8 for the
  // upper four k of a step, + 16 for the second step) and dims 32 dt +
  // 16 ((lane / 16) % 2) + 4 (lane % 4)
  uint32_t rofs[KS], tofs[NDT];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    rofs[s] = static_cast<uint32_t>(l32 * D + 8 * ((2 * s + h32) ^ dqt_swz<NC>(l32))) * 2u;
  {
    const int s16 = lane & 15, g2 = (lane >> 4) & 1;
    const int vr = 4 * h32 + (s16 >> 2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int vc = 4 * dt + 2 * g2 + ((s16 & 3) >> 1);
      tofs[dt] = static_cast<uint32_t>(vr * D + 8 * (vc ^ dqt_swz<NC>(vr)) + 4 * (s16 & 1)) * 2u;
    }
  }
  // K^T operand of dim tile dt, k-step t2: keys 16 t2 + 4 h32 + {0..3, 8..11},
  // the order in which S^T's accumulator holds them (B operand straight from it)
  // rows 8 further: the same positions with bit 1 flipped (NC = 16), bit 1
  // of this lane's position being bit 1 of its chunk, (lane / 16) % 2
  const int tdel = NC >= 16 ? (((lane >> 4) & 1) ? -32 : 32) : 0;
  auto kread = [&](uint32_t slot, int dt, int t2) __attribute__((always_inline)) {
    const char* p = raw + slot + tofs[dt] + t2 * 16 * D * 2;
    const v4s v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(p));
    const v4s v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(p + 8 * D * 2 + tdel));
    return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  };

  float dsum = 0.f, dlt = 0.f;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  const int kt_first = ts.kmin >> 5, kt_last = ts.kmax >> 5;

  auto sweep = [&](auto passc) __attribute__((always_inline)) {
    constexpr bool kDq = decltype(passc)::value;
    for (int seg0 = kt_first; seg0 <= kt_last; seg0 += kSegTiles) {
      const int nseg = min(kSegTiles, kt_last - seg0 + 1);
      // the previous segment's tiles, masks and slots are no longer read
      __syncthreads();
      for (int i = tid; i < BQ * nseg; i += 256) {
        const int qi = i / nseg, j = i - qi * nseg;
        const int tq = qa + qi;
        mask[qi][j] = tq < a.S_q ? qbits[route_row(a, b, tq, kvh) * qwords + seg0 + j] : 0u;
      }
      __syncthreads();
      // compact list of the key tiles any query routes to
      if (wid == 0) {
        int base = 0;
        for (int j0 = 0; j0 < kSegTiles; j0 += 64) {
          const int j = j0 + lane;
          uint32_t any = 0u;
          if (j < nseg)
            for (int qi = 0; qi < BQ; ++qi) any |= mask[qi][j];
          const uint64_t bal = __ballot(any != 0u);
          if (any) tiles[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
          base += __popcll(bal);
        }
        if (lane == 0) s_ntiles = base;
      }
      __syncthreads();
      const int ntiles = s_ntiles;
      if (ntiles == 0) continue;
      issue(seg0 + tiles[0], 0);
      for (int i = 0; i < ntiles; ++i) {
        const int cur = i & 1;
        // tile i's loads (the only ones in flight) have landed; past the
        // barrier every wave is done with tile i - 1, whose slot is refilled
        __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
        bare_barrier();
        if (i + 1 < ntiles) issue(seg0 + tiles[i + 1], cur ^ 1);
        const uint32_t slot = static_cast<uint32_t>(cur) * BUF;
        const char* kb = raw + slot;
        const char* vb = raw + slot + KBYTES;
        const uint32_t mw = mask[colq][tiles[i]] >> (4 * h32);
        f32x16 st, dpt;
#pragma unroll
        for (int e = 0; e < 16; ++e) { st[e] = 0.f; dpt[e] = 0.f; }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kb + rofs[s]), qop[s], st, 0, 0, 0);
          dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vb + rofs[s]), dop[s], dpt, 0, 0, 0);
        }
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int bit = 8 * (e >> 2) + (e & 3);
          p[e] = ((mw >> bit) & 1u) ? exp2f(st[e] * sc2 - lse2) : 0.f;
        }
        if constexpr (!kDq) {
#pragma unroll
          for (int e = 0; e < 16; ++e) dsum += p[e] * dpt[e];
        } else {
          float ds[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) ds[e] = p[e] * (dpt[e] - dlt);
          const bf16x8 dsb[2] = {pack_bf16x8(ds), pack_bf16x8(ds + 8)};
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(slot, dt, t2), dsb[t2], acc[dt], 0, 0, 0);
        }
      }
    }
  };
  if (have_delta) {
    // Delta given (from the forward's FP32 output): the second sweep only
    dlt = tok ? delta[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] : 0.f;
  } else {
    sweep(std::false_type{});
    // the column's two lane halves hold different keys
    const uint32_t u = __float_as_uint(dsum);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    dlt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  sweep(std::true_type{});

  // ---- epilogue: this lane holds dims 32 dt + 8 j + 4 h32 + {0..3} of its column
  if (tok) {
    if (h32 == 0 && !have_delta) delta[(static_cast<int64_t>(b) * a.Hq + hh) * a.S_q + t] = dlt;
    T* op = dq + ((static_cast<int64_t>(b) * a.S_q + t) * a.Hq + hh) * D + 4 * h32;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v[4] = {acc[dt][4 * j] * a.scale, acc[dt][4 * j + 1] * a.scale, acc[dt][4 * j + 2] * a.scale,
                            acc[dt][4 * j + 3] * a.scale};
        bstore4(op + 32 * dt + 8 * j, v);
      }
  }
}

// ---------------------------------------------------------------- dk / dv
constexpr int kListCap = 128;
constexpr int kRedChunk = 8;   // accumulator slices summed across the waves per LDS round

// One workgroup per (16-key tile, KV head); its four waves take every fourth
// 64-candidate chunk of the tile's reverse list, and their dK / dV partial
// sums meet in LDS before wave 0 stores them.
template <typename T, int D, int DV>
__global__ void __launch_bounds__(256)
bwd_dkdv_kernel(AttnBwdArgs args, const float* __restrict__ delta, const T* __restrict__ qt, const T* __restrict__ dot,
                int G, int Gp, int nkt, int n_items, int merged) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int KS = D / 32, VS = DV / 32, NDK = D / 16, NDV = DV / 16;
  __shared__ int s_t[4][kListCap];
  __shared__ uint32_t s_m[4][kListCap];
  __shared__ f32x4 s_red[3][kRedChunk][64];
  const AttnArgs& a = args.f;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int kvh = item % a.Hkv;
  const int jt = (item / a.Hkv) % nkt;
  const int b = item / (a.Hkv * nkt);
  const int k0 = 16 * jt;
  const int kid = k0 + l16;
  const bool kok = kid < a.S_k;
  const T* kr = static_cast<const T*>(a.k) + b * a.sk_b + static_cast<int64_t>(kok ? kid : 0) * a.sk_t + kvh * a.sk_h + 8 * g16;
  const T* vr = static_cast<const T*>(a.v) + b * a.sv_b + static_cast<int64_t>(kok ? kid : 0) * a.sv_t + kvh * a.sv_h + 8 * g16;
  const T* dout = static_cast<const T*>(args.dout);

  f32x4 adk[NDK], adv[NDV];
#pragma unroll
  for (int i = 0; i < NDK; ++i) adk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NDV; ++i) adv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc2 = a.scale * kLog2eB;
  const int qpb = Gp <= 32 ? 32 / Gp : 1;       // queries per 32-row batch
  const int bpq = Gp <= 32 ? 1 : Gp / 32;       // batches per query

  // one 32-row batch over list slots [s0, s0 + qpb) of this wave's LDS list
  // (slots at or past nv are empty), head block hb when a query spans batches
  auto batch = [&](int s0, int nv, int hb) __attribute__((always_inline)) {
    auto tq = [&](int slot) -> int { return slot < nv ? s_t[wid][s0 + slot] : -1; };
    auto mq = [&](int slot) -> uint32_t { return slot < nv ? s_m[wid][s0 + slot] : 0u; };
    f32x4 sacc[2], pacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + l16;
      const int slot = Gp <= 32 ? r / Gp : 0;
      const int h = Gp <= 32 ? r % Gp : hb * 32 + r;
      const int tr = tq(slot);
      const bool ok = tr >= 0 && h < G;      // this lane's A row is a (query, head) row
      const int hh = kvh * G + (h < G ? h : 0);
      const int tt = tr >= 0 ? tr : 0;
      const T* qp = static_cast<const T*>(a.q) + b * a.sq_b + static_cast<int64_t>(tt) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * g16;
      const T* dp = dout + ((static_cast<int64_t>(b) * a.S_q + tt) * a.Hq + hh) * DV + 8 * g16;
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 xh, xl, yh, yl;
        bld8(qp + 32 * s, xh, xl);
        bld8(kr + 32 * s, yh, yl);
        if (!ok) { bzero8(xh); bzero8(xl); }
        sacc[rt] = bmma<kSplit>(xh, xl, yh, yl, sacc[rt]);
      }
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        bf16x8 xh, xl, yh, yl;
        bld8(dp + 32 * s, xh, xl);
        bld8(vr + 32 * s, yh, yl);
        if (!ok) { bzero8(xh); bzero8(xl); }
        pacc[rt] = bmma<kSplit>(xh, xl, yh, yl, pacc[rt]);
      }
    }
    // P and dS for rows 16rt + 4g16 + i, key l16
    float p[2][4], ds[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g16 + i;
        const int slot = Gp <= 32 ? r / Gp : 0;
        const int h = Gp <= 32 ? r % Gp : hb * 32 + r;
        const int tr = tq(slot);
        float pv = 0.f, dv = 0.f;
        if (tr >= 0 && h < G && ((mq(slot) >> l16) & 1u)) {
          const int64_t li = (static_cast<int64_t>(b) * a.Hq + kvh * G + h) * a.S_q + tr;
          pv = exp2f(sacc[rt][i] * sc2 - args.lse[li] * kLog2eB);
          dv = pv * (pacc[rt][i] - delta[li]);
        }
        p[rt][i] = pv;
        ds[rt][i] = dv;
      }
    // P and dS always go in as bf16 high + low halves: dK and dV sum these
    // products over every query routed to the key, so operand rounding would
    // accumulate; with the split the sums are FP32-accurate.
    bf16x8 ph, pl, sh, sl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bput_f(ph, pl, j, p[0][j], true);
      bput_f(ph, pl, 4 + j, p[1][j], true);
      bput_f(sh, sl, j, ds[0][j], true);
      bput_f(sh, sl, 4 + j, ds[1][j], true);
    }
    // A operands: rows rho(g16, j) = 4g16 + j (j < 4) and 16 + 4g16 + (j - 4)
    const int rA = 4 * g16, rB = 16 + 4 * g16;
    const int sA = Gp <= 32 ? rA / Gp : 0, sB = Gp <= 32 ? rB / Gp : 0;
    const int hA = Gp <= 32 ? rA % Gp : hb * 32 + rA, hB = Gp <= 32 ? rB % Gp : hb * 32 + rB;
    const int tA = tq(sA), tB = tq(sB);
    const int64_t baseA = (static_cast<int64_t>(b) * a.S_q + (tA >= 0 ? tA : 0)) * a.Hkv + kvh;
    const int64_t baseB = (static_cast<int64_t>(b) * a.S_q + (tB >= 0 ? tB : 0)) * a.Hkv + kvh;
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt) {
      const int d = dt * 16 + l16;
      bf16x8 xh, xl;
      bzero8(xh); bzero8(xl);
      if (tA >= 0) bld4(dot + baseA * DV * Gp + static_cast<int64_t>(d) * Gp + hA, xh, xl, 0);
      if (tB >= 0) bld4(dot + baseB * DV * Gp + static_cast<int64_t>(d) * Gp + hB, xh, xl, 4);
      adv[dt] = bmma_split_b<kSplit>(xh, xl, ph, pl, adv[dt]);
    }
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      const int d = dt * 16 + l16;
      bf16x8 xh, xl;
      bzero8(xh); bzero8(xl);
      if (tA >= 0) bld4(qt + baseA * D * Gp + static_cast<int64_t>(d) * Gp + hA, xh, xl, 0);
      if (tB >= 0) bld4(qt + baseB * D * Gp + static_cast<int64_t>(d) * Gp + hB, xh, xl, 4);
      adk[dt] = bmma_split_b<kSplit>(xh, xl, sh, sl, adk[dt]);
    }
  };

  // walk the reverse list: listed query tiles, every query inside them (lists
  // of the route group read by this KV head: [RG, B, key tiles, width])
  const int64_t lrow = (static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b) * nkt + jt;
  const int cnt = args.rev_counts[lrow];
  const int32_t* qtiles = args.rev_indices + lrow * args.rev_width;
  const int bq = args.rev_bq;
  const int64_t ncand = static_cast<int64_t>(cnt) * bq;
  int listed = 0;   // entries in s_t/s_m waiting for a batch
  for (int64_t c0 = 64 * wid; c0 < ncand; c0 += 256) {
    const int64_t cidx = c0 + lane;
    int t = -1;
    uint32_t mask = 0u;
    if (cidx < ncand) {
      const int qtile = qtiles[cidx / bq];
      t = qtile * bq + static_cast<int>(cidx % bq);
      if (qtile < 0 || t >= a.S_q) t = -1;
    }
    if (t >= 0) {
      const int64_t qrow = route_row(a, b, t, kvh);
      const int n = max(0, min(a.lens[qrow], a.L));
      const int32_t* r = a.routes + qrow * a.L;
      int lo = 0, hi = n;                 // first entry >= k0
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (r[mid] < k0) lo = mid + 1; else hi = mid;
      }
      for (int e = lo; e < n; ++e) {
        const int id = r[e];
        if (id >= k0 + 16) break;
        if (id >= k0) mask |= 1u << (id - k0);
      }
    }
    const bool hit = mask != 0u;
    const uint64_t bal = __ballot(hit);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (hit) {
      s_t[wid][listed + before] = t;
      s_m[wid][listed + before] = mask;
    }
    listed += __popcll(bal);
    wave_lds_sync();
    // drain full batches
    int used = 0;
    while (listed - used >= qpb) {
      for (int hb = 0; hb < bpq; ++hb) batch(used, qpb, hb);
      used += qpb;
    }
    // keep the remainder at the front
    const int rem = listed - used;
    int keep_t = -1;
    uint32_t keep_m = 0u;
    if (lane < rem) { keep_t = s_t[wid][used + lane]; keep_m = s_m[wid][used + lane]; }
    wave_lds_sync();
    if (lane < rem) { s_t[wid][lane] = keep_t; s_m[wid][lane] = keep_m; }
    listed = rem;
    wave_lds_sync();
  }
  if (listed > 0) {
    for (int hb = 0; hb < bpq; ++hb) batch(0, listed, hb);
  }

  // waves 1-3 hand their partial sums to wave 0, kRedChunk slices at a time
  // (slice s < NDK is adk[s], the rest adv[s - NDK]); fixed summation order
  constexpr int NS = NDK + NDV;
#pragma unroll
  for (int c = 0; c < NS; c += kRedChunk) {
    if (wid > 0) {
#pragma unroll
      for (int j = 0; j < kRedChunk; ++j)
        if (c + j < NS) s_red[wid - 1][j][lane] = c + j < NDK ? adk[c + j < NDK ? c + j : 0] : adv[c + j >= NDK ? c + j - NDK : 0];
    }
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int j = 0; j < kRedChunk; ++j) {
        if (c + j >= NS) continue;
        const f32x4 w = s_red[0][j][lane] + s_red[1][j][lane] + s_red[2][j][lane];
        if (c + j < NDK) adk[c + j < NDK ? c + j : 0] += w;
        else adv[c + j >= NDK ? c + j - NDK : 0] += w;
      }
    }
    __syncthreads();
  }

  if (wid != 0 || !kok) return;
  T* dkp = static_cast<T*>(args.dk) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * D + 4 * g16;
  if (merged) {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = adk[dt][i] * a.scale + (dt < NDV ? adv[dt < NDV ? dt : 0][i] : 0.f);
      bstore4(dkp + dt * 16, v);
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      const float v[4] = {adk[dt][0] * a.scale, adk[dt][1] * a.scale, adk[dt][2] * a.scale, adk[dt][3] * a.scale};
      bstore4(dkp + dt * 16, v);
    }
    T* dvp = static_cast<T*>(args.dv) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * DV + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt) {
      const float v[4] = {adv[dt][0], adv[dt][1], adv[dt][2], adv[dt][3]};
      bstore4(dvp + dt * 16, v);
    }
  }
}

// ---------------------------------------------------------------- hit lists
// 16-bit mask of the keys [k0, k0 + 16) in query t's ascending route; gb =
// g * B + b picks batch row b of route group g
IRB_DEV uint32_t route_tile_mask(const AttnArgs& a, int gb, int t, int k0) {
  const int64_t qrow = static_cast<int64_t>(gb) * a.S_q + t;
  const int n = max(0, min(a.lens[qrow], a.L));
  const int32_t* r = a.routes + qrow * a.L;
  int lo = 0, hi = n;                 // first entry >= k0
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (r[mid] < k0) lo = mid + 1; else hi = mid;
  }
  // the tile's keys are among the (at most 16) entries from lo on: their
  // loads are independent and issue together
  uint32_t m = 0u;
  const int e1 = min(n, lo + 16);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lo + i;
    const int id = e < e1 ? r[e] : -1;
    m |= (id >= k0 && id < k0 + 16) ? 1u << (id - k0) : 0u;
  }
  return m;
}

// One workgroup per (route group, b, key tile).  pass 0 counts the reverse-list queries
// whose route holds a key of the tile; pass 1 writes them, ascending, with
// their key masks from hit_off[tile] on (never past cap).  With one query per
// reverse-list row (rev_bq = 1) every listed query is a hit by construction,
// so pass 0 only copies the list's count and pass 1 places each query at its
// list position with no search-dependent scan (a listed query whose route
// misses the tile, possible only with a stale list, gets mask 0 and adds
// nothing to dK / dV).
__global__ void __launch_bounds__(256)
bwd_hits_kernel(AttnBwdArgs args, int nkt, int pass, int64_t* __restrict__ hit_off, int32_t* __restrict__ hit_t,
                uint32_t* __restrict__ hit_m, int64_t cap) {
  __shared__ int wsum[4];
  const AttnArgs& a = args.f;
  const int64_t lrow = blockIdx.x;
  const int gb = static_cast<int>(lrow / nkt), j = static_cast<int>(lrow % nkt);
  const int k0 = 16 * j;
  const int cnt = min(max(args.rev_counts[lrow], 0), args.rev_width);
  const int32_t* qtiles = args.rev_indices + lrow * args.rev_width;
  const int bq = args.rev_bq;
  const int64_t ncand = static_cast<int64_t>(cnt) * bq;
  const int64_t base = pass ? hit_off[lrow] : 0;
  const int64_t end = pass ? min(hit_off[lrow + 1], cap) : 0;
  if (bq == 1) {
    if (!pass) {
      if (threadIdx.x == 0) hit_off[lrow] = cnt;
      return;
    }
    for (int c = threadIdx.x; c < cnt; c += 256) {
      const int64_t pos = base + c;
      if (pos >= end) break;
      const int qt = qtiles[c];
      const bool ok = qt >= 0 && qt < a.S_q;
      hit_t[pos] = ok ? qt : -1;
      hit_m[pos] = ok ? route_tile_mask(a, gb, qt, k0) : 0u;
    }
    return;
  }
  int64_t done = 0;
  for (int64_t c0 = 0; c0 < ncand; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    int t = -1;
    uint32_t m = 0u;
    if (c < ncand) {
      const int qt = qtiles[c / bq];
      const int64_t tt = static_cast<int64_t>(qt) * bq + c % bq;
      if (qt >= 0 && tt < a.S_q) {
        t = static_cast<int>(tt);
        m = route_tile_mask(a, gb, t, k0);
      }
    }
    int tot;
    const int incl = block_scan256(m != 0u ? 1 : 0, wsum, &tot);
    if (pass && m != 0u) {
      const int64_t pos = base + done + incl - 1;
      if (pos < end) {
        hit_t[pos] = t;
        hit_m[pos] = m;
      }
    }
    done += tot;
  }
  if (!pass && threadIdx.x == 0) hit_off[lrow] = done;
}

// in-place exclusive prefix sum of v[0, n); v[n] receives the total and
// *dropped (when given) the hits beyond the capacity, which the filling pass
// cannot store
__global__ void __launch_bounds__(256)
bwd_scan_kernel(int64_t* __restrict__ v, int64_t n, int64_t cap, int64_t* __restrict__ dropped) {
  __shared__ int64_t part[256];
  const int tid = threadIdx.x;
  const int64_t per = (n + 255) / 256;
  const int64_t lo = min(n, static_cast<int64_t>(tid) * per), hi = min(n, lo + per);
  int64_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += v[i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t x = part[i];
      part[i] = run;
      run += x;
    }
    v[n] = run;
    if (dropped) *dropped = run > cap ? run - cap : 0;
  }
  __syncthreads();
  int64_t run = part[tid];
  for (int64_t i = lo; i < hi; ++i) {
    const int64_t x = v[i];
    v[i] = run;
    run += x;
  }
}

// ---------------------------------------------------------------- union hit lists
// Hit lists of 64-key groups (four consecutive 16-key tiles) for the shared-
// batch mode of the key side.  One workgroup per (route group, b, group): the
// queries of the group's four tile lists (entries with a non-zero key mask)
// are marked in an LDS bitmap over the row's S_q queries; pass 0 counts
// them, pass 1 writes them ascending from off64[group] on (never past cap64)
// with the four tiles' 16-bit masks side by side (0 where a tile's list lacks
// the query).  LDS: the bitmap, then (pass 1) each word's exclusive count.
__global__ void __launch_bounds__(256)
bwd_union_kernel(int S_q, int nkt, int ngrp, int pass, const int64_t* __restrict__ hit_off,
                 const int32_t* __restrict__ hit_t, const uint32_t* __restrict__ hit_m, int64_t cap,
                 int64_t* __restrict__ off64, int32_t* __restrict__ t64, uint16_t* __restrict__ m64, int64_t cap64) {
  extern __shared__ uint32_t ub[];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int words = (S_q + 31) / 32;
  uint32_t* bm = ub;
  int* pre = reinterpret_cast<int*>(ub + words);
  const int64_t grow = blockIdx.x;
  const int64_t gb = grow / ngrp;
  const int J = static_cast<int>(grow % ngrp);
  const int64_t lrow0 = gb * nkt + 4 * J;
  const int ntl = min(4, nkt - 4 * J);
  for (int i = tid; i < words; i += 256) bm[i] = 0u;
  __syncthreads();
  for (int w = 0; w < ntl; ++w) {
    const int64_t h0 = min(hit_off[lrow0 + w], cap), h1 = min(hit_off[lrow0 + w + 1], cap);
    for (int64_t e = h0 + tid; e < h1; e += 256) {
      const int t = hit_t[e];
      if (t >= 0 && t < S_q && hit_m[e] != 0u) atomicOr(&bm[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  if (pass == 0) {
    int c = 0;
    for (int i = tid; i < words; i += 256) c += __popc(bm[i]);
    int tot;
    block_scan256(c, wsum, &tot);
    if (tid == 0) off64[grow] = tot;
    return;
  }
  const int64_t base = min(off64[grow], cap64), end = min(off64[grow + 1], cap64);
  int run = 0;
  for (int w0 = 0; w0 < words; w0 += 256) {
    const int i = w0 + tid;
    const uint32_t x = i < words ? bm[i] : 0u;
    const int pc = __popc(x);
    int tot;
    const int incl = block_scan256(pc, wsum, &tot);
    int o = run + incl - pc;
    if (i < words) pre[i] = o;
    uint32_t y = x;
    while (y) {
      const int bit = __ffs(y) - 1;
      y &= y - 1;
      const int64_t pos = base + o++;
      if (pos < end) {
        t64[pos] = i * 32 + bit;
        *reinterpret_cast<uint2*>(m64 + 4 * pos) = make_uint2(0u, 0u);
      }
    }
    run += tot;
  }
  // the zeroed masks are in place before the tiles' fields are written
  __syncthreads();
  for (int w = 0; w < ntl; ++w) {
    const int64_t h0 = min(hit_off[lrow0 + w], cap), h1 = min(hit_off[lrow0 + w + 1], cap);
    for (int64_t e = h0 + tid; e < h1; e += 256) {
      const int t = hit_t[e];
      const uint32_t m = hit_m[e];
      if (t < 0 || t >= S_q || m == 0u) continue;
      const int64_t pos = base + pre[t >> 5] + __popc(bm[t >> 5] & ((1u << (t & 31)) - 1u));
      if (pos < end) m64[4 * pos + w] = static_cast<uint16_t>(m);
    }
  }
}

// ---------------------------------------------------------------- dk / dv over hit lists
// Whether 64-key group J of (b, KV head kvh) runs in shared batches: its
// four 16-key tile lists hold at least overlap_milli / 1000 times as many
// entries as their union (off64 == nullptr: no union lists, never).  Every
// wave of both key-side launches evaluates the same counts.
IRB_DEV bool union_group(const AttnArgs& a, int b, int kvh, int J, int nkt, int ngrp,
                         const int64_t* __restrict__ hit_off, int64_t cap, const int64_t* __restrict__ off64,
                         int64_t cap64, int overlap_milli) {
  if (off64 == nullptr) return false;
  const int64_t g = static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b;
  const int64_t lrow64 = g * ngrp + J;
  const int64_t u = min(off64[lrow64 + 1], cap64) - min(off64[lrow64], cap64);
  const int64_t l0 = g * nkt + 4 * J, l1 = g * nkt + min(4 * J + 4, nkt);
  const int64_t sumc = min(hit_off[l1], cap) - min(hit_off[l0], cap);
  return u > 0 && u * overlap_milli <= sumc * 1000;
}

// Dispatch order of the key-side workgroups, heaviest first: item (b, group,
// KV head) weighs its union count when it runs in shared batches, else its
// longest tile list (the slowest of its four waves); items go out by
// descending half-octave bucket of that weight, in their launch order inside
// a bucket (neighbouring groups share window queries through the L2).  One
// workgroup; every workgroup of the key side writes its own key tiles only,
// so the order changes no result, only how the long lists spread over the chip.
constexpr int kOrderMax = 1 << 16;   // larger grids keep the launch order
__global__ void __launch_bounds__(1024)
bwd_order_kernel(AttnArgs a, int nkt, const int64_t* __restrict__ hit_off, int64_t cap,
                 const int64_t* __restrict__ off64, int64_t cap64, int overlap_milli, int32_t* __restrict__ ord) {
  constexpr int NBK = 64, NW = 16;
  __shared__ int cnt[NBK];
  __shared__ int wc[NW][NBK];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ngrp = (nkt + 3) / 4;
  const int items = a.B * ngrp * a.Hkv;
  if (threadIdx.x < NBK) cnt[threadIdx.x] = 0;
  __syncthreads();
  auto bucket = [&](int it) -> int {
    const int kvh = it % a.Hkv, J = (it / a.Hkv) % ngrp, b = it / (a.Hkv * ngrp);
    const int64_t g = static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b;
    int64_t w = 0;
    if (union_group(a, b, kvh, J, nkt, ngrp, hit_off, cap, off64, cap64, overlap_milli)) {
      w = min(off64[g * ngrp + J + 1], cap64) - min(off64[g * ngrp + J], cap64);
    } else {
      for (int j = 4 * J; j < min(4 * J + 4, nkt); ++j)
        w = max(w, min(hit_off[g * nkt + j + 1], cap) - min(hit_off[g * nkt + j], cap));
    }
    const uint64_t w1 = static_cast<uint64_t>(w) + 1;
    const int lg = 63 - __clzll(w1);                                   // floor(log2(w + 1))
    const int k = 2 * lg + (lg > 0 ? static_cast<int>((w1 >> (lg - 1)) & 1) : 0);
    return NBK - 1 - min(k, NBK - 1);
  };
  for (int it = threadIdx.x; it < items; it += blockDim.x) atomicAdd(&cnt[bucket(it)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < NBK; ++k) {
      const int c = cnt[k];
      cnt[k] = run;
      run += c;
    }
  }
  __syncthreads();
  // stable scatter, 1024 items at a time: rank inside the wave by ballot,
  // then after the same bucket's items of the lower waves
  for (int c0 = 0; c0 < items; c0 += NW * 64) {
    const int it = c0 + static_cast<int>(threadIdx.x);
    const int k = it < items ? bucket(it) : -1;
    int rank = 0;
    for (int kk = 0; kk < NBK; ++kk) {
      const uint64_t m = __ballot(k == kk);
      if (k == kk) rank = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) wc[wid][kk] = __popcll(m);
    }
    __syncthreads();
    if (k >= 0) {
      int pos = cnt[k] + rank;
      for (int w = 0; w < wid; ++w) pos += wc[w][k];
      ord[pos] = it;
    }
    __syncthreads();
    if (threadIdx.x < NBK) {
      int t = 0;
      for (int w = 0; w < NW; ++w) t += wc[w][threadIdx.x];
      cnt[threadIdx.x] += t;
    }
    __syncthreads();
  }
}


// LDS of a shared-batch group: four batch buffers, each the batch's q and dO
// rows (32 rows of D bf16 each) + lse, Delta, masks and the next ids
template <int D>
constexpr int union_lds_bytes() {
  return 4 * (2 * 32 * D * 2 + 256 + 64 + 32);
}
template <int D, int DV, int GP>
IRB_DEV void dkdv_union_group(const AttnBwdArgs& args, const float* __restrict__ delta, int G, int nkt, int merged,
                              const int64_t* __restrict__ off64, const int32_t* __restrict__ t64,
                              const uint16_t* __restrict__ m64, int64_t cap64, char* lds, int item);

// GP > 0: the padded group size as a constant (4, 8, 16, 32: the row ->
// (query, head) splits below become shifts and masks); 0: Gp_rt at run time.
// With union lists (off64), a workgroup whose group passes union_group runs
// it in shared batches (dkdv_union_group) in the same launch, so the long
// lists of either kind overlap with the other kind's groups.
template <int D, int DV, int GP>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_hits_kernel(AttnBwdArgs args, const float* __restrict__ delta, const int64_t* __restrict__ hit_off,
                     const int32_t* __restrict__ hit_t, const uint32_t* __restrict__ hit_m, int64_t cap, int G,
                     int Gp_rt, int nkt, int merged, const int64_t* __restrict__ off64, const int32_t* __restrict__ t64,
                     const uint16_t* __restrict__ m64, int64_t cap64, int overlap_milli,
                     const int32_t* __restrict__ ord) {
  constexpr int KS = D / 32, VS = DV / 32, NDK = D / 16, NDV = DV / 16;
  const int Gp = GP > 0 ? GP : Gp_rt;
  // row pitches of the slabs: 8 dwords apart modulo 64 banks, so the 8-byte
  // words of 8 consecutive rows land in distinct banks
  constexpr int LQ = D + 16, LO = DV + 16;
  constexpr int kSlabs = 4 * 32 * (LQ + LO) * 2;
  constexpr int kLds = GP > 0 && union_lds_bytes<D>() > kSlabs ? union_lds_bytes<D>() : kSlabs;
  __shared__ __align__(16) char lds[kLds];
  auto s_q = reinterpret_cast<uint16_t(*)[32 * LQ]>(lds);
  auto s_o = reinterpret_cast<uint16_t(*)[32 * LO]>(lds + 4 * 32 * LQ * 2);
  const AttnArgs& a = args.f;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  // one workgroup per (b, four consecutive 16-key tiles, KV head), wave w on
  // tile 4 J + w: neighbouring tiles' lists share queries (a window, dense
  // routes), whose q / dO rows the four waves then find in the L2
  const int ngrp = (nkt + 3) / 4;
  // (b, group, KV head) of this workgroup: heaviest first when ordered
  const int item = ord ? ord[blockIdx.x] : static_cast<int>(blockIdx.x);
  const int kvh = item % a.Hkv;
  const int J = (item / a.Hkv) % ngrp;
  const int b = item / (a.Hkv * ngrp);
  const int jt = 4 * J + wid;
  // groups whose tile lists overlap enough run in shared batches
  if (GP > 0 && union_group(a, b, kvh, J, nkt, ngrp, hit_off, cap, off64, cap64, overlap_milli)) {
    if constexpr (GP > 0) dkdv_union_group<D, DV, GP>(args, delta, G, nkt, merged, off64, t64, m64, cap64, lds, item);
    return;
  }
  if (jt >= nkt) return;
  const int k0 = 16 * jt;
  const int kid = k0 + l16;
  const bool kok = kid < a.S_k;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* og = static_cast<const uint16_t*>(args.dout);

  // the tile's keys and values as B operands: key l16, dims 8 g16 + 32 s
  bf16x8 kb[KS], vb[VS];
  {
    const uint16_t* kr = static_cast<const uint16_t*>(a.k) + b * a.sk_b + static_cast<int64_t>(kok ? kid : 0) * a.sk_t +
                         kvh * a.sk_h + 8 * g16;
    const uint16_t* vr = static_cast<const uint16_t*>(a.v) + b * a.sv_b + static_cast<int64_t>(kok ? kid : 0) * a.sv_t +
                         kvh * a.sv_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kb[s] = *reinterpret_cast<const bf16x8*>(kr + 32 * s);
      if (!kok) bzero8(kb[s]);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      vb[s] = *reinterpret_cast<const bf16x8*>(vr + 32 * s);
      if (!kok) bzero8(vb[s]);
    }
  }
  f32x4 adk[NDK], adv[NDV];
#pragma unroll
  for (int i = 0; i < NDK; ++i) adk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NDV; ++i) adv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc2 = a.scale * kLog2eB;
  const int qpb = Gp <= 32 ? 32 / Gp : 1;       // queries per 32-row batch
  const int bpq = Gp <= 32 ? 1 : Gp / 32;       // batches per query
  const int64_t lrow = (static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b) * nkt + jt;
  const int64_t h0 = min(hit_off[lrow], cap), h1 = min(hit_off[lrow + 1], cap);
  uint16_t* sq = s_q[wid];
  uint16_t* so = s_o[wid];
  // this lane's word for the transpose reads: row 4 g16 + l16 / 4, column 4 (l16 % 4)
  const int tr_off_q = (4 * g16 + (l16 >> 2)) * LQ + 4 * (l16 & 3);
  const int tr_off_o = (4 * g16 + (l16 >> 2)) * LO + 4 * (l16 & 3);

  // Hit ids of a batch (hb-th 32-row part of the hits from e0 on): hit_t of
  // this lane's two A rows (16 rt + l16), and for each row tile rt hit_t /
  // hit_m of the query holding the lane's softmax rows 16 rt + 4 g16 .. + 3
  // (with Gp >= 4 those four rows belong to one query).  They are loaded one
  // batch ahead, so a batch waits for one round of loads: its q / dO rows
  // together with its lse and Delta values.
  // The raw list entries with their validity (checked where they are used,
  // so the loads have no consumer in the fetching iteration and stay in
  // flight; masking them at fetch time had the compiler wait for them there)
  struct Ids {
    int ta[2], ts[2];
    uint32_t tm[2];
    bool va[2], vs[2];
  };
  // (branch-free: entries past the list read its first entry, a valid
  // address, and are then discarded)
  auto fetch = [&](int64_t e0_, int hb_, Ids& d) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + l16;
      const int slot = Gp <= 32 ? r / Gp : 0;
      const int h = Gp <= 32 ? r % Gp : hb_ * 32 + r;
      const int64_t e = e0_ + slot;
      d.ta[rt] = hit_t[e < h1 ? e : h0];
      d.va[rt] = e < h1 && h < G;
      const int rs = 16 * rt + 4 * g16;
      const int64_t es = e0_ + (Gp <= 32 ? rs / Gp : 0);
      d.ts[rt] = hit_t[es < h1 ? es : h0];
      d.tm[rt] = hit_m[es < h1 ? es : h0];
      d.vs[rt] = es < h1;
    }
  };
  // Second half of a batch: P and dS at rows 16 rt + 4 g16 + i, key l16
  // (zero off the key mask) as bf16 high/low operands (form_pds), then
  // dV^T += dO^T P and dK^T += Q^T dS with the A operands read transposed
  // from the slabs written by start (accumulate).  k-slot j of the A
  // operands is row 4 g16 + j (j < 4) or 16 + 4 g16 + (j - 4), matching P / dS.
  struct PdS {
    bf16x8 ph, pl, sh, sl;
  };
  auto form_pds = [&](const f32x4 (&sacc)[2], const f32x4 (&pacc)[2], const float (&lsv)[2][4],
                      const float (&dlv)[2][4], const bool (&rok)[2][4], PdS& o) __attribute__((always_inline)) {
    float p[2][4], ds[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // every lane evaluates the exponential (no branch per element);
        // masked entries are then replaced by 0 (their inputs may come
        // from the stand-in row)
        const float e = fast_exp2(sacc[rt][i] * sc2 - lsv[rt][i] * kLog2eB);
        p[rt][i] = rok[rt][i] ? e : 0.f;
        ds[rt][i] = rok[rt][i] ? e * (pacc[rt][i] - dlv[rt][i]) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bput_f(o.ph, o.pl, j, p[0][j], true);
      bput_f(o.ph, o.pl, 4 + j, p[1][j], true);
      bput_f(o.sh, o.sl, j, ds[0][j], true);
      bput_f(o.sh, o.sl, 4 + j, ds[1][j], true);
    }
  };
  // The NDV + NDK dim tiles run as one sequence (dV tiles, then dK tiles)
  // whose transposed A operands are read kAhead tiles ahead of their MFMAs,
  // so several LDS reads are in flight behind each pair of MFMAs.
  constexpr int kAhead = 3;
  auto tile_operand = [&](int u) __attribute__((always_inline)) {
    const uint16_t* w = u < NDV ? so + tr_off_o + 16 * u : sq + tr_off_q + 16 * (u - NDV);
    const int pitch = u < NDV ? LO : LQ;
    const v4s x0 = lds_read_tr(w), x1 = lds_read_tr(w + 16 * pitch);
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto accumulate = [&](const PdS& o) __attribute__((always_inline)) {
    wave_lds_sync();
    bf16x8 xa[kAhead + 1];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) xa[u] = tile_operand(u);
#pragma unroll
    for (int u = 0; u < NDV + NDK; ++u) {
      if (u + kAhead < NDV + NDK) xa[(u + kAhead) % (kAhead + 1)] = tile_operand(u + kAhead);
      const bf16x8 x = xa[u % (kAhead + 1)];
      if (u < NDV) {
        adv[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.ph, adv[u], 0, 0, 0);
        adv[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.pl, adv[u], 0, 0, 0);
      } else {
        adk[u - NDV] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.sh, adk[u - NDV], 0, 0, 0);
        adk[u - NDV] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.sl, adk[u - NDV], 0, 0, 0);
      }
    }
    wave_lds_sync();   // the slabs are rewritten by the next batch
  };
  // First half of a batch: the rows' copies into the slabs and S = Q K^T,
  // dP = dO V^T
  auto start = [&](const bf16x8 (&qa)[2][KS], const bf16x8 (&oa)[2][VS], f32x4 (&sacc)[2],
                   f32x4 (&pacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<bf16x8*>(sq + (16 * rt + l16) * LQ + 8 * g16 + 32 * s) = qa[rt][s];
#pragma unroll
      for (int s = 0; s < VS; ++s)
        *reinterpret_cast<bf16x8*>(so + (16 * rt + l16) * LO + 8 * g16 + 32 * s) = oa[rt][s];
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      pacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][s], kb[s], sacc[rt], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < VS; ++s) pacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[rt][s], vb[s], pacc[rt], 0, 0, 0);
    }
  };
  // Rows of the batch at e0_ (ids d, 32-row part hb_) in the A layout
  auto load_rows = [&](int64_t e0_, int hb_, const Ids& d, bf16x8 (&qa)[2][KS], bf16x8 (&oa)[2][VS])
                       __attribute__((always_inline)) {
    // every row of the batch a real (query, head): no row needs zeroing
    const bool full = e0_ + qpb <= h1 && G == Gp;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + l16;
      const int h = Gp <= 32 ? r % Gp : hb_ * 32 + r;
      const int t = d.va[rt] && d.ta[rt] < a.S_q ? d.ta[rt] : -1;
      const int hh = kvh * G + (h < G ? h : 0);
      const int tt = t >= 0 ? t : 0;
      const uint16_t* qp = qg + b * a.sq_b + static_cast<int64_t>(tt) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * g16;
      const uint16_t* op = og + ((static_cast<int64_t>(b) * a.S_q + tt) * a.Hq + hh) * DV + 8 * g16;
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[rt][s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
#pragma unroll
      for (int s = 0; s < VS; ++s) oa[rt][s] = *reinterpret_cast<const bf16x8*>(op + 32 * s);
      if (!full && t < 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) bzero8(qa[rt][s]);
#pragma unroll
        for (int s = 0; s < VS; ++s) bzero8(oa[rt][s]);
      }
    }
  };
  // lse / Delta / key-mask flags of the batch's softmax rows (index 0 stands
  // in for rows without a query; their weights are zeroed in finish)
  auto load_stats = [&](int hb_, const Ids& d, float (&lsv)[2][4], float (&dlv)[2][4], bool (&rok)[2][4])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g16 + i;
        const int h = Gp <= 32 ? r % Gp : hb_ * 32 + r;
        const int te = d.vs[rt] && d.ts[rt] < a.S_q ? d.ts[rt] : -1;
        rok[rt][i] = te >= 0 && h < G && ((d.tm[rt] >> l16) & 1u);
        const int64_t li = rok[rt][i] ? (static_cast<int64_t>(b) * a.Hq + kvh * G + h) * a.S_q + te : 0;
        lsv[rt][i] = args.lse[li];
        dlv[rt][i] = delta[li];
      }
  };

  if constexpr (GP > 0) {
    // one 32-row batch per qpb listed queries (bpq = 1), software-pipelined:
    // the rows and statistics of batch e0 + qpb load into the registers
    // batch e0 has just released (rows after its S and dP, statistics after
    // its P and dS) while batch e0's dK / dV work runs, and the ids of the
    // batch after that are read meanwhile
    bf16x8 qa[2][KS], oa[2][VS];
    float lsv[2][4], dlv[2][4];
    bool rok[2][4];
    Ids nxt;
    if (h0 < h1) {
      Ids cur;
      fetch(h0, 0, cur);
      load_rows(h0, 0, cur, qa, oa);
      load_stats(0, cur, lsv, dlv, rok);
      if (h0 + qpb < h1) fetch(h0 + qpb, 0, nxt);
    }
    for (int64_t e0 = h0; e0 < h1; e0 += qpb) {
      f32x4 sacc[2], pacc[2];
      start(qa, oa, sacc, pacc);
      PdS o;
      form_pds(sacc, pacc, lsv, dlv, rok, o);
      // The next rows are issued only after P and dS have consumed this
      // batch's statistics: memory-operation counters complete in order, so
      // a wait for the statistics placed after these loads would wait for
      // them too.  The empty statement uses the operands and orders memory.
      asm volatile("" : : "v"(o.ph), "v"(o.pl), "v"(o.sh), "v"(o.sl) : "memory");
      const int64_t ne0 = e0 + qpb;
      if (ne0 < h1) {
        load_rows(ne0, 0, nxt, qa, oa);
        load_stats(0, nxt, lsv, dlv, rok);
        if (ne0 + qpb < h1) fetch(ne0 + qpb, 0, nxt);
      }
      accumulate(o);
    }
  } else {
    // run-time group size (G > 32: several 32-row batches per query)
    Ids cur;
    if (h0 < h1) fetch(h0, 0, cur);
    for (int64_t e0 = h0; e0 < h1; e0 += qpb) {
      for (int hb = 0; hb < bpq; ++hb) {
        bf16x8 qa[2][KS], oa[2][VS];
        float lsv[2][4], dlv[2][4];
        bool rok[2][4];
        load_rows(e0, hb, cur, qa, oa);
        load_stats(hb, cur, lsv, dlv, rok);
        // the next batch's ids
        Ids nxt;
        {
          const int64_t ne0 = hb + 1 < bpq ? e0 : e0 + qpb;
          const int nhb = hb + 1 < bpq ? hb + 1 : 0;
          if (ne0 < h1) fetch(ne0, nhb, nxt);
        }
        f32x4 sacc[2], pacc[2];
        start(qa, oa, sacc, pacc);
        PdS o;
        form_pds(sacc, pacc, lsv, dlv, rok, o);
        accumulate(o);
        cur = nxt;
      }
    }
  }

  if (!kok) return;
  uint16_t* dkp = static_cast<uint16_t*>(args.dk) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * D + 4 * g16;
  if (merged) {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = adk[dt][i] * a.scale + (dt < NDV ? adv[dt < NDV ? dt : 0][i] : 0.f);
      bstore4(dkp + dt * 16, v);
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      const float v[4] = {adk[dt][0] * a.scale, adk[dt][1] * a.scale, adk[dt][2] * a.scale, adk[dt][3] * a.scale};
      bstore4(dkp + dt * 16, v);
    }
    uint16_t* dvp = static_cast<uint16_t*>(args.dv) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * DV + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt) {
      const float v[4] = {adv[dt][0], adv[dt][1], adv[dt][2], adv[dt][3]};
      bstore4(dvp + dt * 16, v);
    }
  }
}

// ---------------------------------------------------------------- dk / dv in shared batches

// 16-byte chunk position of chunk c of row r in a shared-batch row buffer:
// c ^ f(r & 15), f a bit permutation (row bits 0-2 to bits 1-3, bit 3 to
// bit 0), so that the A-operand reads of 16 consecutive rows at one chunk
// and the 32-lane transpose reads of eight consecutive rows at two
// neighbouring chunks both hit distinct banks (rows are 256 bytes, whole
// bank rounds, so without it they would not; 128-byte rows use three bits)
template <int NC>
IRB_DEV int ub_pos(int r, int c) {
  const int f = NC > 8 ? (((r & 7) << 1) | ((r >> 3) & 1)) : (((r & 3) << 1) | ((r >> 2) & 1));
  return c ^ f;
}

// Groups of four 16-key tiles whose lists overlap (union_group), run by the
// workgroup of bwd_dkdv_hits_kernel that the group falls to (b, group, KV
// head), wave w on tile 4 J + w with its keys and values as B operands as in
// the per-tile path.  The group's union list
// runs in batches of QPB queries (32 rows); each batch's q and dO rows, the
// rows' lse and Delta and the queries' key masks go by direct global-to-LDS
// loads into one of four buffers, three batches ahead of the one being
// computed, so a workgroup keeps three batches of loads in flight; each
// batch's loads also bring the query ids of the batch three later, which
// address that batch's loads once this one has landed.  Every
// wave applies its own tile to each batch (skipping batches that reach none
// of its keys) exactly as the per-tile kernel does, so the sums differ only
// in the order of their terms.
template <int D, int DV, int GP>
IRB_DEV void dkdv_union_group(const AttnBwdArgs& args, const float* __restrict__ delta, int G, int nkt, int merged,
                              const int64_t* __restrict__ off64, const int32_t* __restrict__ t64,
                              const uint16_t* __restrict__ m64, int64_t cap64, char* lds, int item) {
  static_assert(D == DV && GP >= 4 && GP <= 32, "shared batches: one row layout, whole queries per batch");
  constexpr int KS = D / 32, VS = DV / 32, NDK = D / 16, NDV = DV / 16;
  constexpr int QPB = 32 / GP;               // queries per batch
  constexpr int NC = D / 8;                  // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int QB = 32 * RB;                // a batch's q rows (then its dO rows)
  constexpr int SB = 2 * QB + 256 + 64 + 32; // + lse[32], Delta[32], masks (2 words per query), ids of batch + 3
  constexpr int NBUF = 4;
  constexpr int NRI = 2 * 32 * NC / 256;     // 16-byte row loads per wave and batch
  static_assert(NRI >= 1 && (2 * 32 * NC) % 256 == 0, "row loads");
  static_assert(NBUF * SB == union_lds_bytes<D>(), "buffer layout");
  const AttnArgs& a = args.f;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int g16 = lane >> 4, l16 = lane & 15;
  const int ngrp = (nkt + 3) / 4;
  const int kvh = item % a.Hkv;
  const int J = (item / a.Hkv) % ngrp;
  const int b = item / (a.Hkv * ngrp);
  const int jt = 4 * J + wid;
  const bool live = jt < nkt;
  const int k0 = 16 * jt;
  const int kid = k0 + l16;
  const bool kok = kid < a.S_k;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* og = static_cast<const uint16_t*>(args.dout);
  const int64_t lrow64 = (static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b) * ngrp + J;
  const int64_t u0 = min(off64[lrow64], cap64), u1 = min(off64[lrow64 + 1], cap64);
  const int nb = static_cast<int>((u1 - u0 + QPB - 1) / QPB);

  bf16x8 kb[KS], vb[VS];
  {
    const uint16_t* kr = static_cast<const uint16_t*>(a.k) + b * a.sk_b + static_cast<int64_t>(kok ? kid : 0) * a.sk_t +
                         kvh * a.sk_h + 8 * g16;
    const uint16_t* vr = static_cast<const uint16_t*>(a.v) + b * a.sv_b + static_cast<int64_t>(kok ? kid : 0) * a.sv_t +
                         kvh * a.sv_h + 8 * g16;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      kb[s2] = *reinterpret_cast<const bf16x8*>(kr + 32 * s2);
      if (!kok) bzero8(kb[s2]);
    }
#pragma unroll
    for (int s2 = 0; s2 < VS; ++s2) {
      vb[s2] = *reinterpret_cast<const bf16x8*>(vr + 32 * s2);
      if (!kok) bzero8(vb[s2]);
    }
  }
  f32x4 adk[NDK], adv[NDV];
#pragma unroll
  for (int i = 0; i < NDK; ++i) adk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NDV; ++i) adv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc2 = a.scale * kLog2eB;

  // row loads: load n of this wave fills 16-byte slots (wv NRI + n) 64 + lane
  // of the buffer; slot s < 32 NC is position s % NC of q row s / NC, the
  // rest the same of the dO rows; row r is head r % GP of the batch's query r / GP
  int rk[NRI], rh[NRI], rc[NRI];
#pragma unroll
  for (int n = 0; n < NRI; ++n) {
    const int slot = (wv * NRI + n) * 64 + lane;
    const int rs = slot % (32 * NC);
    const int r = rs / NC;
    rk[n] = r / GP;
    rh[n] = r % GP;
    rc[n] = ub_pos<NC>(r, rs % NC);          // the global chunk stored at this position (f is an involution)
  }
  const uint32_t lds0 = lds_addr(lds);
  // a batch's query ids as one vector value (registers)
  typedef int TQ __attribute__((ext_vector_type(8)));
  static_assert(QPB <= 8, "ids per batch");
  auto tpick = [&](TQ tq, int k) __attribute__((always_inline)) {
    int t = tq[0];
#pragma unroll
    for (int kk = 1; kk < QPB; ++kk) t = k == kk ? tq[kk] : t;
    return t;
  };
  // query ids of batch j from memory (the first batches; entries past the list repeat its last)
  auto load_t = [&](int j) __attribute__((always_inline)) {
    const int64_t e0 = u0 + static_cast<int64_t>(j) * QPB;
    TQ tq = TQ{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < QPB; ++kk) {
      const int64_t e = e0 + kk < u1 ? e0 + kk : u1 - 1;
      tq[kk] = t64[e];
    }
    return tq;
  };
  auto issue = [&](int j, TQ tq) __attribute__((always_inline)) {
    const int64_t e0 = u0 + static_cast<int64_t>(j) * QPB;
    const uint32_t base = lds0 + static_cast<uint32_t>(j % NBUF) * SB;
#pragma unroll
    for (int n = 0; n < NRI; ++n) {
      const bool ok = e0 + rk[n] < u1 && rh[n] < G;
      const int t = ok ? tpick(tq, rk[n]) : 0;
      const int hh = kvh * G + (rh[n] < G ? rh[n] : 0);
      const bool isq = (wv * NRI + n) * 64 < 32 * NC;       // wave-uniform
      const uint16_t* src = isq ? qg + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * rc[n]
                                : og + ((static_cast<int64_t>(b) * a.S_q + t) * a.Hq + hh) * DV + 8 * rc[n];
      lds_dma16(src, base + (wv * NRI + n) * 1024);
    }
    if (wv == 0) {
      // lse (lanes 0-31) and Delta (lanes 32-63) of the batch's 32 rows
      const int r = lane & 31, k = r / GP, h = r % GP;
      const bool ok = e0 + k < u1 && h < G;
      const int64_t li = ok ? (static_cast<int64_t>(b) * a.Hq + kvh * G + h) * a.S_q + tpick(tq, k) : 0;
      lds_dma4(lane < 32 ? args.lse + li : delta + li, base + 2 * QB);
    } else if (wv == 1) {
      // the queries' four 16-bit tile masks (two words each)
      if (lane < 2 * QPB) {
        const int64_t e = e0 + (lane >> 1) < u1 ? e0 + (lane >> 1) : u1 - 1;
        lds_dma4(m64 + 4 * e + 2 * (lane & 1), base + 2 * QB + 256);
      }
    } else if (wv == 2) {
      // the query ids of batch j + NBUF - 1
      if (lane < QPB) {
        const int64_t en = e0 + (NBUF - 1) * QPB + lane;
        lds_dma4(t64 + (en < u1 ? en : u1 - 1), base + 2 * QB + 320);
      }
    }
  };

  // P and dS of a batch as bf16 high / low operands (as in the per-tile kernel)
  struct PdS {
    bf16x8 ph, pl, sh, sl;
  };
  auto tile_operand = [&](const char* buf, int u) __attribute__((always_inline)) {
    const bool isv = u < NDV;
    const char* rows = isv ? buf + QB : buf;
    const int uu = isv ? u : u - NDV;
    const int r = 4 * g16 + (l16 >> 2);
    const int c = 2 * uu + ((l16 & 3) >> 1);
    const char* p = rows + r * RB + 16 * ub_pos<NC>(r, c) + 8 * (l16 & 1);
    const v4s x0 = lds_read_tr(reinterpret_cast<const uint16_t*>(p));
    const v4s x1 = lds_read_tr(reinterpret_cast<const uint16_t*>(p + 16 * RB));   // row r + 16: same f
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  constexpr int kAhead = 3;

  if (nb > 0) {
    const int npre = nb < NBUF - 1 ? nb : NBUF - 1;
    for (int j = 0; j < npre; ++j) issue(j, load_t(j));
    for (int i = 0; i < nb; ++i) {
      // batch i's loads (this wave's) have landed once only the later
      // batches' may still be out; then the barrier publishes every wave's
      // (waves 0-2 issue one load per batch more than wave 3)
      const int later = min(NBUF - 2, nb - 1 - i);
      if (later <= 0) __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
      else if (later == 1) {
        if (wv < 3) __builtin_amdgcn_s_waitcnt(kDmaWait<NRI + 1>());
        else __builtin_amdgcn_s_waitcnt(kDmaWait<NRI>());
      } else {
        if (wv < 3) __builtin_amdgcn_s_waitcnt(kDmaWait<2 * (NRI + 1)>());
        else __builtin_amdgcn_s_waitcnt(kDmaWait<2 * NRI>());
      }
      bare_barrier();
      const char* buf = lds + (i % NBUF) * SB;
      // every wave is done with batch i - 1: its buffer takes batch i + 3,
      // addressed by the ids that batch i brought
      if (i + NBUF - 1 < nb) {
        const int* tn = reinterpret_cast<const int*>(buf + 2 * QB + 320);
        TQ tq = TQ{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < QPB; ++kk) tq[kk] = tn[kk];
        issue(i + NBUF - 1, tq);
      }
      const float* st = reinterpret_cast<const float*>(buf + 2 * QB);
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(buf + 2 * QB + 256);
      const int64_t e0 = u0 + static_cast<int64_t>(i) * QPB;
      float lsv[2][4], dlv[2][4];
      bool rok[2][4];
      int any = 0;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int k = (16 * rt + 4 * g16) / GP;
        const uint32_t m16 = (mw[2 * k + (wid >> 1)] >> (16 * (wid & 1))) & 0xffffu;
        const bool qok = e0 + k < u1 && ((m16 >> l16) & 1u);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = 16 * rt + 4 * g16 + i4;
          rok[rt][i4] = qok && (r % GP) < G;
          lsv[rt][i4] = st[r];
          dlv[rt][i4] = st[32 + r];
          any |= rok[rt][i4] ? 1 : 0;
        }
      }
      // a wave none of whose keys the batch reaches skips it
      if (live && __ballot(any) != 0ull) {
        f32x4 sacc[2], pacc[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          pacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int r = 16 * rt + l16;
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2)
            sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *reinterpret_cast<const bf16x8*>(buf + r * RB + 16 * ub_pos<NC>(r, g16 + 4 * s2)), kb[s2], sacc[rt], 0, 0, 0);
#pragma unroll
          for (int s2 = 0; s2 < VS; ++s2)
            pacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *reinterpret_cast<const bf16x8*>(buf + QB + r * RB + 16 * ub_pos<NC>(r, g16 + 4 * s2)), vb[s2], pacc[rt], 0,
                0, 0);
        }
        PdS o;
        {
          float p[2][4], ds[2][4];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const float e = fast_exp2(sacc[rt][i4] * sc2 - lsv[rt][i4] * kLog2eB);
              p[rt][i4] = rok[rt][i4] ? e : 0.f;
              ds[rt][i4] = rok[rt][i4] ? e * (pacc[rt][i4] - dlv[rt][i4]) : 0.f;
            }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bput_f(o.ph, o.pl, j, p[0][j], true);
            bput_f(o.ph, o.pl, 4 + j, p[1][j], true);
            bput_f(o.sh, o.sl, j, ds[0][j], true);
            bput_f(o.sh, o.sl, 4 + j, ds[1][j], true);
          }
        }
        bf16x8 xa[kAhead + 1];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) xa[u] = tile_operand(buf, u);
#pragma unroll
        for (int u = 0; u < NDV + NDK; ++u) {
          if (u + kAhead < NDV + NDK) xa[(u + kAhead) % (kAhead + 1)] = tile_operand(buf, u + kAhead);
          const bf16x8 x = xa[u % (kAhead + 1)];
          if (u < NDV) {
            adv[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.ph, adv[u], 0, 0, 0);
            adv[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.pl, adv[u], 0, 0, 0);
          } else {
            adk[u - NDV] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.sh, adk[u - NDV], 0, 0, 0);
            adk[u - NDV] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, o.sl, adk[u - NDV], 0, 0, 0);
          }
        }
      }
    }
  }

  if (!kok) return;
  uint16_t* dkp = static_cast<uint16_t*>(args.dk) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * D + 4 * g16;
  if (merged) {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = adk[dt][r] * a.scale + (dt < NDV ? adv[dt < NDV ? dt : 0][r] : 0.f);
      bstore4(dkp + dt * 16, v);
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
      const float v[4] = {adk[dt][0] * a.scale, adk[dt][1] * a.scale, adk[dt][2] * a.scale, adk[dt][3] * a.scale};
      bstore4(dkp + dt * 16, v);
    }
    uint16_t* dvp = static_cast<uint16_t*>(args.dv) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * DV + 4 * g16;
#pragma unroll
    for (int dt = 0; dt < NDV; ++dt) {
      const float v[4] = {adv[dt][0], adv[dt][1], adv[dt][2], adv[dt][3]};
      bstore4(dvp + dt * 16, v);
    }
  }
}

// ---------------------------------------------------------------- dk / dv, latent width
// D = 576, Dv = 512, heads in whole 32-row batches.  One 256-thread workgroup
// per (16-key tile, KV head), one listed query at a time: waves 0 and 1 load
// the batch's 32 q rows (16 each) into the A layout, keep the tile's keys as
// B operands and form S; waves 2 and 3 do the same with dO rows, values and
// dP.  Both row sets also go row-major into LDS slabs, S and dP through a
// small LDS exchange; then every wave forms P and dS for all 32 rows and owns
// every fourth 16-dim tile of dK^T += q^T dS and dV^T += dO^T P, reading the
// transposed A operands from the slabs.
template <int D, int DV>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_wide_kernel(AttnBwdArgs args, const float* __restrict__ delta, const int64_t* __restrict__ hit_off,
                     const int32_t* __restrict__ hit_t, const uint32_t* __restrict__ hit_m, int64_t cap, int G,
                     int nkt, int merged) {
  constexpr int KS = D / 32, VS = DV / 32, NDK = D / 16, NDV = DV / 16;
  constexpr int MK = (NDK + 3) / 4, MV = (NDV + 3) / 4;   // dim tiles per wave
  // slab pitches: rows 40 (q, 296 dwords) and 8 (dO, 264 dwords) banks apart, so
  // the 8-byte words of 8 consecutive rows never share a bank
  constexpr int LQ = D + 16, LO = DV + 16;
  static_assert(KS >= VS, "key width below value width");
  __shared__ __align__(16) uint16_t s_q[32 * LQ];
  __shared__ __align__(16) uint16_t s_o[32 * LO];
  __shared__ f32x4 s_x[4][64];          // S rows 0-15, S rows 16-31, dP rows 0-15, dP rows 16-31
  const AttnArgs& a = args.f;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int item = blockIdx.x;
  const int kvh = item % a.Hkv;
  const int jt = (item / a.Hkv) % nkt;
  const int b = item / (a.Hkv * nkt);
  const int k0 = 16 * jt;
  const int kid = k0 + l16;
  const bool kok = kid < a.S_k;
  const bool is_s = wid < 2;            // waves 0, 1: S from q and K; waves 2, 3: dP from dO and V
  const int rt = wid & 1;               // this wave's 16 of the batch's 32 rows

  bf16x8 kb[KS];
  {
    const uint16_t* src = is_s
        ? static_cast<const uint16_t*>(a.k) + b * a.sk_b + static_cast<int64_t>(kok ? kid : 0) * a.sk_t + kvh * a.sk_h
        : static_cast<const uint16_t*>(a.v) + b * a.sv_b + static_cast<int64_t>(kok ? kid : 0) * a.sv_t + kvh * a.sv_h;
    const int ns = is_s ? KS : VS;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s < ns && kok) kb[s] = *reinterpret_cast<const bf16x8*>(src + 8 * g16 + 32 * s);
      else bzero8(kb[s]);
    }
  }
  f32x4 adk[MK], adv[MV];
#pragma unroll
  for (int i = 0; i < MK; ++i) adk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MV; ++i) adv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc2 = a.scale * kLog2eB;
  const int bpq = G / 32;
  const int64_t lrow = (static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b) * nkt + jt;
  const int64_t h0 = min(hit_off[lrow], cap), h1 = min(hit_off[lrow + 1], cap);
  const int tr_row = 4 * g16 + (l16 >> 2), tr_col = 4 * (l16 & 3);
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* og = static_cast<const uint16_t*>(args.dout);

  // the next hit's query and key mask are read one hit ahead
  int nt = h0 < h1 ? hit_t[h0] : -1;
  uint32_t nm = h0 < h1 ? hit_m[h0] : 0u;
  for (int64_t e = h0; e < h1; ++e) {
    const int t = nt;
    const uint32_t m = nm;
    if (e + 1 < h1) {
      nt = hit_t[e + 1];
      nm = hit_m[e + 1];
    }
    if (t < 0 || t >= a.S_q) continue;          // uniform over the workgroup
    const bool kin = (m >> l16) & 1u;
    for (int hb = 0; hb < bpq; ++hb) {
      {
        const int hh = kvh * G + hb * 32 + 16 * rt + l16;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if (is_s) {
          const uint16_t* src = qg + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t + static_cast<int64_t>(hh) * a.sq_h + 8 * g16;
          bf16x8 xa[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s) xa[s] = *reinterpret_cast<const bf16x8*>(src + 32 * s);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            *reinterpret_cast<bf16x8*>(s_q + (16 * rt + l16) * LQ + 8 * g16 + 32 * s) = xa[s];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], kb[s], acc, 0, 0, 0);
          }
        } else {
          const uint16_t* src = og + ((static_cast<int64_t>(b) * a.S_q + t) * a.Hq + hh) * DV + 8 * g16;
          bf16x8 xa[VS];
#pragma unroll
          for (int s = 0; s < VS; ++s) xa[s] = *reinterpret_cast<const bf16x8*>(src + 32 * s);
#pragma unroll
          for (int s = 0; s < VS; ++s) {
            *reinterpret_cast<bf16x8*>(s_o + (16 * rt + l16) * LO + 8 * g16 + 32 * s) = xa[s];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], kb[s], acc, 0, 0, 0);
          }
        }
        s_x[wid][lane] = acc;
      }
      // lse and Delta of rows 16 r2 + 4 g16 + i, loaded before the exchange
      float lsv[2][4], dlv[2][4];
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t li = (static_cast<int64_t>(b) * a.Hq + kvh * G + hb * 32 + 16 * r2 + 4 * g16 + i) * a.S_q + t;
          lsv[r2][i] = args.lse[li];
          dlv[r2][i] = delta[li];
        }
      __syncthreads();
      // P and dS at rows 16 r2 + 4 g16 + i, key l16
      float p[2][4], ds[2][4];
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const f32x4 sv = s_x[r2][lane], pv = s_x[2 + r2][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pp = kin ? exp2f(sv[i] * sc2 - lsv[r2][i] * kLog2eB) : 0.f;
          p[r2][i] = pp;
          ds[r2][i] = kin ? pp * (pv[i] - dlv[r2][i]) : 0.f;
        }
      }
      bf16x8 ph, pl, sh, sl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bput_f(ph, pl, j, p[0][j], true);
        bput_f(ph, pl, 4 + j, p[1][j], true);
        bput_f(sh, sl, j, ds[0][j], true);
        bput_f(sh, sl, 4 + j, ds[1][j], true);
      }
#pragma unroll
      for (int i = 0; i < MK; ++i) {
        const int dt = wid + 4 * i;
        if (dt < NDK) {
          const uint16_t* w = s_q + tr_row * LQ + tr_col + 16 * dt;
          const v4s x0 = lds_read_tr(w), x1 = lds_read_tr(w + 16 * LQ);
          const bf16x8 xa = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          adk[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, sh, adk[i], 0, 0, 0);
          adk[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, sl, adk[i], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < MV; ++i) {
        const int dt = wid + 4 * i;
        if (dt < NDV) {
          const uint16_t* w = s_o + tr_row * LO + tr_col + 16 * dt;
          const v4s x0 = lds_read_tr(w), x1 = lds_read_tr(w + 16 * LO);
          const bf16x8 xa = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          adv[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ph, adv[i], 0, 0, 0);
          adv[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, pl, adv[i], 0, 0, 0);
        }
      }
      __syncthreads();   // slabs and the exchange are rewritten by the next batch
    }
  }

  if (!kok) return;
  uint16_t* dkp = static_cast<uint16_t*>(args.dk) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * D + 4 * g16;
#pragma unroll
  for (int i = 0; i < MK; ++i) {
    const int dt = wid + 4 * i;
    if (dt >= NDK) continue;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = adk[i][r] * a.scale;
    // wave w's i-th value tile is tile w + 4 i too, so the merged sum stays in-lane
    if (merged && i < MV && dt < NDV) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += adv[i][r];
    }
    bstore4(dkp + dt * 16, v);
  }
  if (!merged) {
    uint16_t* dvp = static_cast<uint16_t*>(args.dv) + ((static_cast<int64_t>(b) * a.S_k + kid) * a.Hkv + kvh) * DV + 4 * g16;
#pragma unroll
    for (int i = 0; i < MV; ++i) {
      const int dt = wid + 4 * i;
      if (dt >= NDV) continue;
      const float v[4] = {adv[i][0], adv[i][1], adv[i][2], adv[i][3]};
      bstore4(dvp + dt * 16, v);
    }
  }
}

template <typename T, int D, int DV>
static int launch_bwd_t(const AttnBwdArgs& args, hipStream_t stream) {
  const AttnArgs& a = args.f;
  const int G = a.Hq / a.Hkv;
  const int Gp = padded_group(G);
  constexpr bool kGqaHits = sizeof(T) == 2 && D == DV && (D == 64 || D == 128);
  constexpr bool kWide = sizeof(T) == 2 && D == 576 && DV == 512;
  const bool hits = kGqaHits || (kWide && G % 32 == 0);
  if constexpr (kWide)
    if (latent_bwd_applies(a, args.dk, args.dv))
      return launch_latent_bwd(a, args.dout, args.lse, args.out32, args.dq, args.dk, args.ws, args.dropped, stream);
  BwdWs ws = carve(args.ws, a.B, a.S_q, a.S_k, a.L, a.Hq, a.Hkv, a.Dqk, a.Dv, a.dtype, a.RG);
  const int latent = (a.v == a.k && a.sv_b == a.sk_b && a.sv_t == a.sk_t && a.sv_h == a.sk_h) ? 1 : 0;
  const int64_t rows = static_cast<int64_t>(a.B) * a.S_q;
  if (!hits) {
    hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, stream, a,
                       static_cast<const T*>(args.dout), static_cast<T*>(ws.qt), static_cast<T*>(ws.dot), G, Gp);
  }
  // query tiles for dQ: key-membership words per route row, kept in the
  // hit-list area of the workspace (the hit lists are built after the dQ pass)
  bool tile_dq = false;
  if constexpr (kGqaHits) {
    const bool small_strides = static_cast<int64_t>(a.sk_t > a.sv_t ? a.sk_t : a.sv_t) * 64 < (int64_t{1} << 31);
    const size_t qb = attn_fwd_qbits_bytes(a);
    const size_t room = 2 * align256(static_cast<size_t>(ws.cap) * 4);
    tile_dq = tile_thr_milli() <= 1000 && small_strides && (G == 4 || G == 8 || G == 16) && qb > 0 && qb <= room;
  }
  // Delta = rowsum(dO o) with o in FP32: read off the forward's FP32 output
  // when given and a pass would otherwise form it (the query-tile dQ, or a
  // forward in Delta mode); else the bf16 query side with G <= 16 forms it
  // in its own pass (written before the key side reads it), and otherwise a
  // forward pass in Delta mode recomputes o
  const bool fused_delta = G <= 16 && dq_fuses_delta<T, D>();
  const bool have_delta = args.out32 != nullptr && (tile_dq || !fused_delta);
  if (have_delta) {
    if (int rc = launch_delta_from_o(a, args.dout, args.out32, ws.delta, stream)) return rc;
  } else if (!fused_delta) {
    if (int rc = launch_attn_delta(a, args.dout, ws.delta, stream)) return rc;
  }
  const int PAD = sizeof(T) == 2 ? 8 : 4;
  const int64_t items = rows * a.Hkv;
  bool dq_done = false;
  int tile_bq = 0;   // > 0: the per-query launch skips the query tiles the tile kernel takes
  if constexpr (kGqaHits) {
    if (tile_dq) {
      uint32_t* qbits = reinterpret_cast<uint32_t*>(ws.hit_t);
      if (int rc = launch_route_bits(a.routes, a.lens, static_cast<int64_t>(a.RG) * rows, a.L, a.S_k, qbits, stream))
        return rc;
      const int qwords = (a.S_k + 31) / 32;
      // routes wide against the key range: nearly every tile is dense, and the
      // tile launch runs the few sparse ones per query itself
      const int gather_rest = static_cast<int64_t>(a.L) * 1000 >= static_cast<int64_t>(tile_thr_milli()) * a.S_k;
      const int BQ = 128 / G;
      const int n_qt = (a.S_q + BQ - 1) / BQ;
      const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * n_qt * a.Hkv));
#define IRB_DQ_TILE(GV)                                                                                        \
  hipLaunchKernelGGL((bwd_dq_tile_kernel<D, GV>), grid, dim3(256), 0, stream, a, static_cast<const uint16_t*>(args.dout), \
                     args.lse, ws.delta, static_cast<uint16_t*>(args.dq), n_qt, tile_thr_milli(), qbits, qwords,   \
                     gather_rest, have_delta ? 1 : 0)
      if (G == 4) IRB_DQ_TILE(4);
      else if (G == 8) IRB_DQ_TILE(8);
      else IRB_DQ_TILE(16);
#undef IRB_DQ_TILE
      dq_done = gather_rest != 0;
      tile_bq = BQ;
    }
  }
  if (dq_done) {
  } else if (G <= 16) {
    const size_t lds = static_cast<size_t>(4) * 32 * (D + PAD) * sizeof(T);
    auto kern = bwd_dq_kernel<T, D, DV, false>;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), lds, stream, a,
                       static_cast<const T*>(args.dout), args.lse, ws.delta, static_cast<T*>(args.dq), G,
                       static_cast<int>(items), latent, gather_head_major(a) ? 1 : 0, tile_bq, tile_thr_milli());
  } else {
    const int slices = (G + 15) / 16;
    const size_t lds = static_cast<size_t>(32) * ((D + PAD) + (latent ? 0 : (DV + PAD))) * sizeof(T);
    auto kern = bwd_dq_kernel<T, D, DV, true>;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return static_cast<int>(e);
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(items)), dim3(64 * slices), lds, stream, a,
                       static_cast<const T*>(args.dout), args.lse, ws.delta, static_cast<T*>(args.dq), G,
                       static_cast<int>(items), latent, 0, 0, 0);
  }
  const int nkt = (a.S_k + 15) / 16;
  const int64_t kitems = static_cast<int64_t>(a.B) * nkt * a.Hkv;
  const int merged = args.dk == args.dv ? 1 : 0;
  if (hits) {
    const int64_t ltiles = static_cast<int64_t>(a.RG) * a.B * nkt;
    hipLaunchKernelGGL(bwd_hits_kernel, dim3(static_cast<unsigned>(ltiles)), dim3(256), 0, stream, args, nkt, 0,
                       ws.hit_off, ws.hit_t, ws.hit_m, ws.cap);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(256), 0, stream, ws.hit_off, ltiles, ws.cap, args.dropped);
    hipLaunchKernelGGL(bwd_hits_kernel, dim3(static_cast<unsigned>(ltiles)), dim3(256), 0, stream, args, nkt, 1,
                       ws.hit_off, ws.hit_t, ws.hit_m, ws.cap);
    if constexpr (kGqaHits) {
      const int ngrp = (nkt + 3) / 4;
      const int64_t lgroups = static_cast<int64_t>(a.RG) * a.B * ngrp;
      if (ws.off64) {
        // union lists of the 64-key groups (count, offsets, fill)
        const size_t lds = static_cast<size_t>((a.S_q + 31) / 32) * 8;
        hipLaunchKernelGGL(bwd_union_kernel, dim3(static_cast<unsigned>(lgroups)), dim3(256), lds, stream, a.S_q, nkt,
                           ngrp, 0, ws.hit_off, ws.hit_t, ws.hit_m, ws.cap, ws.off64, ws.t64, ws.m64, ws.cap64);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(256), 0, stream, ws.off64, lgroups, ws.cap64,
                           static_cast<int64_t*>(nullptr));
        hipLaunchKernelGGL(bwd_union_kernel, dim3(static_cast<unsigned>(lgroups)), dim3(256), lds, stream, a.S_q, nkt,
                           ngrp, 1, ws.hit_off, ws.hit_t, ws.hit_m, ws.cap, ws.off64, ws.t64, ws.m64, ws.cap64);
      }
      // one launch: per-tile groups, and (with union lists) the shared-batch groups
      const int64_t kgroups = static_cast<int64_t>(a.B) * ngrp * a.Hkv;
      const dim3 grid(static_cast<unsigned>(kgroups));
      const int ovl = key_overlap_milli();
      const int32_t* ord = nullptr;
      if (ws.off64 && kgroups <= kOrderMax) {
        hipLaunchKernelGGL(bwd_order_kernel, dim3(1), dim3(1024), 0, stream, a, nkt, ws.hit_off, ws.cap, ws.off64,
                           ws.cap64, ovl, ws.ord);
        ord = ws.ord;
      }
#define IRB_DKDV_HITS(GPV)                                                                                   \
  hipLaunchKernelGGL((bwd_dkdv_hits_kernel<D, DV, GPV>), grid, dim3(256), 0, stream, args, ws.delta, ws.hit_off, \
                     ws.hit_t, ws.hit_m, ws.cap, G, Gp, nkt, merged, ws.off64, ws.t64, ws.m64, ws.cap64, ovl, \
                     ord)
      if (Gp == 4) IRB_DKDV_HITS(4);
      else if (Gp == 8) IRB_DKDV_HITS(8);
      else if (Gp == 16) IRB_DKDV_HITS(16);
      else if (Gp == 32) IRB_DKDV_HITS(32);
      else IRB_DKDV_HITS(0);
#undef IRB_DKDV_HITS
    } else if constexpr (kWide) {
      hipLaunchKernelGGL((bwd_dkdv_wide_kernel<D, DV>), dim3(static_cast<unsigned>(kitems)), dim3(256), 0, stream,
                         args, ws.delta, ws.hit_off, ws.hit_t, ws.hit_m, ws.cap, G, nkt, merged);
    }
  } else {
    // no hit lists on this path: nothing can be dropped
    if (args.dropped)
      if (int rc = launch_fill_i32(reinterpret_cast<int32_t*>(args.dropped), 2, 0, stream)) return rc;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, DV>), dim3(static_cast<unsigned>(kitems)), dim3(256), 0, stream,
                       args, ws.delta, static_cast<const T*>(ws.qt), static_cast<const T*>(ws.dot), G, Gp, nkt,
                       static_cast<int>(kitems), merged);
  }
  return 0;
}

int launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.f.dtype == IRB_BF16) {
    if (a.f.Dqk == 64 && a.f.Dv == 64) return launch_bwd_t<uint16_t, 64, 64>(a, stream);
    if (a.f.Dqk == 128 && a.f.Dv == 128) return launch_bwd_t<uint16_t, 128, 128>(a, stream);
    if (a.f.Dqk == 576 && a.f.Dv == 512) return launch_bwd_t<uint16_t, 576, 512>(a, stream);
  } else {
    if (a.f.Dqk == 64 && a.f.Dv == 64) return launch_bwd_t<float, 64, 64>(a, stream);
    if (a.f.Dqk == 128 && a.f.Dv == 128) return launch_bwd_t<float, 128, 128>(a, stream);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

}  // namespace irb
