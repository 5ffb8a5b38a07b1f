// a6 for shared latent KV: sparse attention of 64 query heads over one
// 576-wide latent row per key (latent page, nemo_automodel...common.
// cudnn_sparse_attention: q [T, 64, 576], kv [T, 1, 576], the value is the
// first 512 channels of the same row; each query attends only to its own
// sorted index list).
//
// One workgroup of four wavefronts per (batch, query, KV head).  Every key's
// row serves all 64 heads (121 flop per gathered byte), so the rows of a
// 16-key chunk are gathered once into LDS by direct global-to-LDS loads,
// NB chunks in flight, and every wavefront reads them from there:
//   S^T[key, head] = K_chunk . Q^T     wave w: heads 16w .. 16w + 15 (16x16x32
//                                       MFMA, A = K rows from LDS, B = its
//                                       query rows, held in registers)
//   softmax                             same wave, one head column per lane;
//                                       P^T (bf16) and the per-head rescale
//                                       factor go to LDS for the next phase
//   O^T[dim, head] += V^T . P^T        wave w: dims 128w .. 128w + 127 of all
//                                       64 heads (32x32x16 MFMA, A = V^T by
//                                       LDS transpose reads, B = P^T)
// One barrier per chunk: the phase after barrier i accumulates chunk i and
// scores chunk i + 1 (P^T is double-buffered), and issues the gather of
// chunk i + NB - 1 into the buffer chunk i - 1 occupied.
// Rows in a buffer are 1152 bytes (72 chunks of 16 bytes); 16-byte chunk c
// of row r is stored at position c ^ (r & 7) so that eight consecutive rows
// read at one logical column, and the four rows of a transpose read, fall
// on distinct banks.
#include <cstdlib>

#include "irb_internal.hpp"

namespace irb {

namespace {

constexpr int kLD = 576, kLDV = 512;      // latent row width, value width
constexpr int kKC = 16;                   // keys per chunk
constexpr int kRowB = kLD * 2;            // bytes per gathered row
constexpr int kRowC = kRowB / 16;         // 16-byte chunks per row (72)
constexpr int kBufB = kKC * kRowB;        // bytes per chunk buffer (18432)
constexpr int kLoads = kBufB / 1024;      // 1024-byte wave loads per chunk (18)
constexpr int kHeads = 64;
constexpr int kPSlot = kHeads * kKC * 2;  // P^T of one chunk: [head][16 keys] bf16
constexpr float kLog2eL = 1.4426950408889634f;
constexpr float kLn2L = 0.6931471805599453f;

// byte offset inside a buffer of (row r, bf16 element d) under the chunk swizzle
IRB_DEV uint32_t swz(int r, int d) {
  return static_cast<uint32_t>(r * kRowB + 16 * ((d >> 3) ^ (r & 7)) + 2 * (d & 7));
}

}  // namespace

// LDS bytes of the latent forward: NB chunk buffers, two P^T slots, two
// rescale rows, the final 1/l row and the Delta partials, then the route.
static size_t latent_fwd_lds(int NB, int L) {
  return static_cast<size_t>(NB) * kBufB + 2 * kPSlot + 2 * kHeads * 4 + kHeads * 4 + 4 * kHeads * 4 +
         static_cast<size_t>(L) * 4;
}

template <int NB, bool kDelta>
__global__ void __launch_bounds__(256, NB <= 3 ? 2 : 1)
latent_fwd_kernel(AttnArgs a, uint16_t* __restrict__ out, float* __restrict__ lse,
                  const uint16_t* __restrict__ dout, float* __restrict__ delta, int n_items) {
  // chunk i + 1 is scored in the phase that accumulates chunk i, so the
  // gather of chunk i + NB - 1 needs NB >= 3 buffers
  static_assert(NB >= 3 && NB <= 4, "chunk buffers");
  extern __shared__ __align__(16) char smem[];
  char* kbuf = smem;
  char* pbuf = smem + NB * kBufB;
  float* alph = reinterpret_cast<float*>(pbuf + 2 * kPSlot);        // [2][64]
  float* linv = alph + 2 * kHeads;                                   // [64]
  float* dpart = linv + kHeads;                                      // [4][64]
  int32_t* ids = reinterpret_cast<int32_t*>(dpart + 4 * kHeads);     // [L]

  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int l16 = lane & 15, g16 = lane >> 4;
  const int l32 = lane & 31, h32 = lane >> 5;
  const QItem it = decode_qitem(item, a.B, a.S_q, a.Hkv, 0);
  const int b = it.b, t = it.t, kvh = it.kvh;
  const int h0 = kvh * kHeads;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const float sc2 = a.scale * kLog2eL;

  // the route, so every lane can address the rows it gathers
  for (int e = tid; e < n; e += 256) ids[e] = route[e];
  // this wave's query rows as S MFMA B operands: column = head l16, k = dims 32 s + 8 g16 ..
  bf16x8 qop[kLD / 32];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t +
                         static_cast<int64_t>(h0 + 16 * wid + l16) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < kLD / 32; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }
  f32x16 oacc[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][hb][i] = 0.f;
  float m2 = -INFINITY, lsum = 0.f;
  const int nch = (n + kKC - 1) / kKC;
  __syncthreads();

  const uint32_t kb0 = lds_addr(kbuf);
  // gather chunk ch into buffer ch % NB: wave w issues loads w, w + 4, ... of
  // the chunk's 18; lane i of load j fills position 64 j + i of the buffer
  auto issue = [&](int ch) __attribute__((always_inline)) {
    const uint32_t dst = kb0 + (ch % NB) * kBufB;
    for (int j = wv; j < kLoads; j += 4) {
      const int p = 64 * j + lane;
      const int r = p / kRowC, pc = p % kRowC;
      const int e = min(kKC * ch + r, n - 1);          // rows past the route repeat its last key
      const int id = ids[e];
      const int ok = (id >= 0 && id < a.S_k) ? id : 0;
      const uint16_t* src = kbase + static_cast<int64_t>(ok) * a.sk_t + 8 * (pc ^ (r & 7));
      lds_dma16(src, dst + 1024 * j);
    }
  };
  // wait until this wave's loads of every chunk but the `later` (0..2) last-issued ones are done
  // (waves below kLoads % 4 issue one load more per chunk)
  auto wait_loads = [&](int later) __attribute__((always_inline)) {
    constexpr int lo = kLoads / 4, hi = kLoads / 4 + 1;
    const bool big = wv < kLoads % 4;
    if (later <= 0) __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
    else if (later == 1) { if (big) __builtin_amdgcn_s_waitcnt(kDmaWait<hi>()); else __builtin_amdgcn_s_waitcnt(kDmaWait<lo>()); }
    else { if (big) __builtin_amdgcn_s_waitcnt(kDmaWait<2 * hi>()); else __builtin_amdgcn_s_waitcnt(kDmaWait<2 * lo>()); }
  };

  // S^T of chunk ch for this wave's heads, then its online softmax: P^T and the
  // rescale factor of every head go to slot ch % 2
  auto score = [&](int ch) __attribute__((always_inline)) {
    const char* kb = kbuf + (ch % NB) * kBufB;
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kLD / 32; ++s) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + swz(l16, 32 * s + 8 * g16));
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[s], st, 0, 0, 0);
    }
    float x[4];
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = kKC * ch + 4 * g16 + j;
      const int id = e < n ? ids[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      x[j] = ok ? st[j] * sc2 : -INFINITY;
      cm = fmaxf(cm, x[j]);
    }
    cm = row4_max(cm);
    // the reference max moves only when a score exceeds it by more than 8
    // (log2 units): weights stay <= 2^8 and rescaling is rare; exact after
    // the final normalisation
    const bool up = cm > m2 + 8.f;
    const float alpha = up ? fast_exp2(m2 - cm) : 1.f;
    m2 = up ? cm : m2;
    const float mref = (m2 == -INFINITY) ? 0.f : m2;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(x[j] - mref);
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    const int slot = ch & 1;
    uint2 pk;
    pk.x = pack_bf16x2(p[0], p[1]);
    pk.y = pack_bf16x2(p[2], p[3]);
    *reinterpret_cast<uint2*>(pbuf + slot * kPSlot + (16 * wid + l16) * (kKC * 2) + 8 * g16) = pk;
    if (g16 == 0) alph[slot * kHeads + 16 * wid + l16] = alpha;
  };

  // O^T += V^T P^T of chunk ch (after the rescale its softmax asked for)
  auto accumulate = [&](int ch) __attribute__((always_inline)) {
    const int slot = ch & 1;
    const float a0 = alph[slot * kHeads + l32], a1 = alph[slot * kHeads + 32 + l32];
    if (__ballot(a0 != 1.f || a1 != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          oacc[dt][0][i] *= a0;
          oacc[dt][1][i] *= a1;
        }
    }
    const char* vb = kbuf + (ch % NB) * kBufB;
    bf16x8 pop[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      pop[hb] = *reinterpret_cast<const bf16x8*>(pbuf + slot * kPSlot + (32 * hb + l32) * (kKC * 2) + 16 * h32);
    // V^T operand (32 dims x 16 keys): 16-lane row g reads keys 8 (g / 2) + {0..3}
    // and + {4..7} of dims 16 (g % 2) + s: lane s addresses key row r0 + s / 4,
    // dims c0 + 4 (s % 4) .. + 3
    const int s16 = lane & 15, g = lane >> 4;
    const int vr = 8 * (g >> 1) + (s16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dcol = 128 * wid + 32 * dt + 16 * (g & 1) + 4 * (s16 & 3);
      const v4s v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb + swz(vr, dcol)));
      const v4s v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb + swz(vr + 4, dcol)));
      const bf16x8 vop = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        oacc[dt][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[hb], oacc[dt][hb], 0, 0, 0);
    }
  };

  if (nch > 0) {
    // prologue: chunks 0 .. NB - 2 in flight, chunk 0 scored
    for (int c = 0; c < NB - 1 && c < nch; ++c) issue(c);
    wait_loads(min(NB - 2, nch - 1));
    __syncthreads();
    score(0);
    for (int i = 0; i < nch; ++i) {
      // chunk i + 1 must have landed (its loads are the oldest still in flight)
      const int later = min(NB - 3, nch - 2 - i);     // chunks issued after i + 1 that may stay in flight
      wait_loads(i + 1 < nch ? later : 0);
      __syncthreads();
      if (i + NB - 1 < nch) issue(i + NB - 1);
      accumulate(i);
      if (i + 1 < nch) score(i + 1);
    }
  }

  // ---- epilogue: per-head sum, lse, 1 / l for the dim-owning waves
  const float ltot = row4_sum(lsum);
  if (g16 == 0) {
    const int h = 16 * wid + l16;
    linv[h] = ltot > 0.f ? 1.f / ltot : 0.f;
    if (!kDelta)
      lse[(static_cast<int64_t>(b) * a.Hq + h0 + h) * a.S_q + t] = ltot > 0.f ? (m2 + log2f(ltot)) * kLn2L : -INFINITY;
  }
  __syncthreads();
  const float i0 = linv[l32], i1 = linv[32 + l32];
  if (kDelta) {
    // Delta[h] = sum_d o[h, d] dO[h, d] with o in FP32: this wave's 128 dims, then the four waves
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const uint16_t* dp = dout + (row * a.Hq + h0 + 32 * hb + l32) * kLDV + 128 * wid + 4 * h32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint2 u = *reinterpret_cast<const uint2*>(dp + 32 * dt + 8 * q4);
          const float d4[4] = {bf16_to_f32(static_cast<uint16_t>(u.x & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(u.x >> 16)),
                               bf16_to_f32(static_cast<uint16_t>(u.y & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(u.y >> 16))};
#pragma unroll
          for (int j = 0; j < 4; ++j) part[hb] += oacc[dt][hb][4 * q4 + j] * d4[j];
        }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const uint32_t u = __float_as_uint(part[hb]);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      part[hb] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (h32 == 0) {
      dpart[wid * kHeads + l32] = part[0] * i0;
      dpart[wid * kHeads + 32 + l32] = part[1] * i1;
    }
    __syncthreads();
    if (tid < kHeads) {
      const float d = (dpart[tid] + dpart[kHeads + tid]) + (dpart[2 * kHeads + tid] + dpart[3 * kHeads + tid]);
      delta[(static_cast<int64_t>(b) * a.Hq + h0 + tid) * a.S_q + t] = d;
    }
    return;
  }
  // o rows: lane holds dims 32 dt + 8 q4 + 4 h32 + {0..3} of head 32 hb + l32
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float inv = hb ? i1 : i0;
    uint16_t* op = out + (row * a.Hq + h0 + 32 * hb + l32) * kLDV + 128 * wid + 4 * h32;
    float* o32 = a.o32 ? a.o32 + (row * a.Hq + h0 + 32 * hb + l32) * kLDV + 128 * wid + 4 * h32 : nullptr;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float v[4] = {oacc[dt][hb][4 * q4] * inv, oacc[dt][hb][4 * q4 + 1] * inv, oacc[dt][hb][4 * q4 + 2] * inv,
                            oacc[dt][hb][4 * q4 + 3] * inv};
        uint2 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * q4) = u;
        if (o32) *reinterpret_cast<float4*>(o32 + 32 * dt + 8 * q4) = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
}

// ================================================================ backward
//
// Gradients of the latent attention, every pass query-major (a query's 64
// heads share each gathered row, so per-key-tile walks that re-gather whole
// query rows for a few live keys are avoided):
//   delta  Delta[h] = rowsum(dO o) with o recomputed in FP32 (the forward
//          kernel in Delta mode)
//   prep   per query, transposed copies of q [dim][head] and dO [dim][head]
//   ds     per query and 16-key chunk: S^T = K Q^T, dP^T = V dO^T (K and V
//          rows gathered into LDS as in the forward), P = exp(S - lse),
//          dS = P (dP - Delta); P and dS written to the pds buffer
//          [query, route slot, (P_hi | P_lo | dS_hi | dS_lo) head] as bf16
//          high and low parts, so the products below keep ~16 significant
//          bits of each (the key-side sums run over thousands of terms)
//   dq     per query: dQ^T += K^T dS^T over its chunks (K^T and dS^T by LDS
//          transpose reads), dq = scale dQ
//   dkv    per query and chunk: dKV[key, :] += scale dS^T q + [P^T dO, 0]
//          with M = the chunk's 16 keys and K = the 64 heads (the transposed
//          copies as B operands, held in registers for the whole query),
//          added to an FP32 accumulator [S_k, 576] by atomic adds
//   final  the FP32 accumulator rounded into the merged bf16 gradient

// gather the 16 latent rows of route slots [16 ch, 16 ch + 16) into a buffer
// (wave w issues loads w, w + 4, ... of the chunk's 18; see the forward)
IRB_DEV void latent_gather(const uint16_t* kbase, int64_t sk_t, int S_k, const int32_t* ids, int n, int ch,
                           uint32_t dst, int wv, int lane) {
  for (int j = wv; j < kLoads; j += 4) {
    const int p = 64 * j + lane;
    const int r = p / kRowC, pc = p % kRowC;
    const int e = min(kKC * ch + r, n - 1);
    const int id = ids[e];
    const int ok = (id >= 0 && id < S_k) ? id : 0;
    lds_dma16(kbase + static_cast<int64_t>(ok) * sk_t + 8 * (pc ^ (r & 7)), dst + 1024 * j);
  }
}

constexpr int kPdsW = 4 * kHeads;          // pds row: P_hi, P_lo, dS_hi, dS_lo (bf16, 64 heads each)

// pds element offset of (route row, slot e)
IRB_DEV int64_t pds_row(int64_t rrow_kv, int L, int e) { return (rrow_kv * L + e) * kPdsW; }

// ---- prep: transposed copies; block = (row, 64-dim slab); slabs 0..8 of q, 9..16 of dO
__global__ void __launch_bounds__(256)
latent_prep_kernel(AttnArgs a, const uint16_t* __restrict__ dout, uint16_t* __restrict__ qt,
                   uint16_t* __restrict__ dot) {
  __shared__ uint16_t tile[64][72];
  const int64_t row = blockIdx.x;                   // (b * S_q + t) * Hkv + kvh
  const int slab = blockIdx.y;
  const int kvh = static_cast<int>(row % a.Hkv);
  const int64_t bt = row / a.Hkv;
  const int b = static_cast<int>(bt / a.S_q), t = static_cast<int>(bt % a.S_q);
  const bool isq = slab < kLD / 64;
  const int d0 = 64 * (isq ? slab : slab - kLD / 64);
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 8; i += 256) {
    const int h = i >> 3, c = i & 7;
    const uint16_t* src = isq ? static_cast<const uint16_t*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t +
                                    static_cast<int64_t>(kvh * kHeads + h) * a.sq_h + d0 + 8 * c
                              : dout + (bt * a.Hq + kvh * kHeads + h) * kLDV + d0 + 8 * c;
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    *reinterpret_cast<uint4*>(&tile[h][8 * c]) = v;
  }
  __syncthreads();
  uint16_t* dst = isq ? qt + (row * kLD + d0) * kHeads : dot + (row * kLDV + d0) * kHeads;
  for (int i = tid; i < 64 * 8; i += 256) {
    const int d = i >> 3, c = i & 7;             // dim d, heads 8 c .. 8 c + 7
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = tile[8 * c + j][d];
    uint4 u;
    u.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
    u.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
    u.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
    u.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(d) * kHeads + 8 * c) = u;
  }
}

// ---- ds: P and dS of every (route slot, head), written to pds
template <int NB>
__global__ void __launch_bounds__(256, 2)
latent_ds_kernel(AttnArgs a, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                 const float* __restrict__ delta, uint16_t* __restrict__ pds, int n_items) {
  extern __shared__ __align__(16) char smem[];
  char* kbuf = smem;
  uint16_t* tl = reinterpret_cast<uint16_t*>(smem + NB * kBufB);        // [2][16 keys][kPdsW]
  int32_t* ids = reinterpret_cast<int32_t*>(smem + NB * kBufB + 2 * kKC * kPdsW * 2);
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int l16 = lane & 15, g16 = lane >> 4;
  const QItem it = decode_qitem(item, a.B, a.S_q, a.Hkv, 0);
  const int b = it.b, t = it.t, kvh = it.kvh;
  const int h0 = kvh * kHeads;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const int64_t prow = row * a.Hkv + kvh;
  const int hd = h0 + 16 * wid + l16;                       // this lane's head
  const float sc2 = a.scale * kLog2eL;
  const int64_t srow = (static_cast<int64_t>(b) * a.Hq + hd) * a.S_q + t;
  const float l2 = lse[srow] * kLog2eL;
  const float dlt = delta[srow];
  for (int e = tid; e < n; e += 256) ids[e] = route[e];
  bf16x8 qop[kLD / 32], dop[kLDV / 32];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.sq_b + static_cast<int64_t>(t) * a.sq_t +
                         static_cast<int64_t>(hd) * a.sq_h + 8 * g16;
#pragma unroll
    for (int s = 0; s < kLD / 32; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
    const uint16_t* dp = dout + (row * a.Hq + hd) * kLDV + 8 * g16;
#pragma unroll
    for (int s = 0; s < kLDV / 32; ++s) dop[s] = *reinterpret_cast<const bf16x8*>(dp + 32 * s);
  }
  const int nch = (n + kKC - 1) / kKC;
  __syncthreads();
  if (nch == 0) return;
  const uint32_t kb0 = lds_addr(kbuf);
  // the 16 x kPdsW tile of chunk ch to pds (two 16-byte pieces per thread)
  auto flush = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pc = tid + 256 * u;
      const int r = pc >> 5, c = pc & 31;
      const int e = kKC * ch + r;
      if (e < n)
        *reinterpret_cast<uint4*>(pds + pds_row(prow, a.L, e) + 8 * c) =
            *reinterpret_cast<const uint4*>(tl + ((ch & 1) * kKC + r) * kPdsW + 8 * c);
    }
  };
  for (int c = 0; c < NB - 1 && c < nch; ++c)
    latent_gather(kbase, a.sk_t, a.S_k, ids, n, c, kb0 + (c % NB) * kBufB, wv, lane);
  for (int i = 0; i < nch; ++i) {
    // chunk i is the oldest load batch in flight; up to NB - 2 later batches may stay
    const int later = min(NB - 2, nch - 1 - i);
    if (later <= 0) __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
    else if (wv < kLoads % 4) __builtin_amdgcn_s_waitcnt(kDmaWait<kLoads / 4 + 1>());
    else __builtin_amdgcn_s_waitcnt(kDmaWait<kLoads / 4>());
    __syncthreads();
    if (i + NB - 1 < nch) latent_gather(kbase, a.sk_t, a.S_k, ids, n, i + NB - 1, kb0 + ((i + NB - 1) % NB) * kBufB, wv, lane);
    if (i > 0) flush(i - 1);
    const char* kb = kbuf + (i % NB) * kBufB;
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f}, dpt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kLD / 32; ++s) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + swz(l16, 32 * s + 8 * g16));
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[s], st, 0, 0, 0);
      if (s < kLDV / 32) dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, dop[s], dpt, 0, 0, 0);
    }
    uint16_t* tw = tl + (i & 1) * kKC * kPdsW;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = kKC * i + 4 * g16 + j;
      const int id = e < n ? ids[e] : -1;
      const bool ok = id >= 0 && id < a.S_k;
      const float p = ok ? fast_exp2(st[j] * sc2 - l2) : 0.f;
      const float ds = p * (dpt[j] - dlt);
      uint16_t ph, pl, dh, dl;
      split_bf16(p, ph, pl);
      split_bf16(ds, dh, dl);
      uint16_t* tr = tw + (4 * g16 + j) * kPdsW + 16 * wid + l16;
      tr[0] = ph;
      tr[kHeads] = pl;
      tr[2 * kHeads] = dh;
      tr[3 * kHeads] = dl;
    }
  }
  __syncthreads();
  flush(nch - 1);
}

// ---- dq: dQ^T += K^T dS^T; wave w owns dim tiles w, w + 4, ... (of 18, 32 dims each)
template <int NB>
__global__ void __launch_bounds__(256, 2)
latent_dq_kernel(AttnArgs a, const uint16_t* __restrict__ pds, uint16_t* __restrict__ dq, int n_items) {
  constexpr int kSB = kKC * kHeads * 2;                     // one dS^T part: [16 keys][64 heads] bf16, 2 KiB
  constexpr int kStage = kBufB + 2 * kSB;                   // K rows, dS_hi, dS_lo
  extern __shared__ __align__(16) char smem[];
  int32_t* ids = reinterpret_cast<int32_t*>(smem + NB * kStage);
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int l32 = lane & 31, h32 = lane >> 5;
  const QItem it = decode_qitem(item, a.B, a.S_q, a.Hkv, 0);
  const int b = it.b, t = it.t, kvh = it.kvh;
  const int h0 = kvh * kHeads;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  const int32_t* route = a.routes + rrow * a.L;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.sk_b + kvh * a.sk_h;
  const int64_t prow = row * a.Hkv + kvh;
  for (int e = tid; e < n; e += 256) ids[e] = route[e];
  constexpr int NT = 5;                                      // dim tiles per wave (18 over 4 waves: 5, 5, 4, 4)
  const int ntw = wid < 2 ? 5 : 4;
  f32x16 acc[NT][2];
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[k][hb][i] = 0.f;
  const int nch = (n + kKC - 1) / kKC;
  __syncthreads();
  const uint32_t sb0 = lds_addr(smem);
  // chunk ch: its K rows (18 loads: 5, 5, 4, 4 by wave) and its dS_hi^T and
  // dS_lo^T rows (2 loads each, by waves 2 and 3, which then issue 6): 16-byte
  // chunk c of key row r at position c ^ (r & 7)
  auto issue = [&](int ch) __attribute__((always_inline)) {
    const uint32_t st0 = sb0 + (ch % NB) * kStage;
    latent_gather(kbase, a.sk_t, a.S_k, ids, n, ch, st0, wv, lane);
    if (wv >= 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = 64 * u + lane;                       // 128 pieces of one part: 16 rows x 8
        const int r = p >> 3, pc = p & 7;
        const int e = min(kKC * ch + r, n - 1);
        lds_dma16(pds + pds_row(prow, a.L, e) + 2 * kHeads + kHeads * (wv - 2) + 8 * (pc ^ (r & 7)),
                  st0 + kBufB + kSB * (wv - 2) + 1024 * u);
      }
    }
  };
  const int s16 = lane & 15, g = lane >> 4;
  const int vr = 8 * (g >> 1) + (s16 >> 2);
  if (nch > 0) {
    for (int c = 0; c < NB - 1 && c < nch; ++c) issue(c);
    for (int i = 0; i < nch; ++i) {
      const int later = min(NB - 2, nch - 1 - i);
      if (later <= 0) __builtin_amdgcn_s_waitcnt(kDmaWait<0>());
      else if (wv < 2) __builtin_amdgcn_s_waitcnt(kDmaWait<5>());
      else __builtin_amdgcn_s_waitcnt(kDmaWait<6>());
      __syncthreads();
      if (i + NB - 1 < nch) issue(i + NB - 1);
      const char* kb = smem + (i % NB) * kStage;
      const char* sb = kb + kBufB;
      // dS^T operands (16 keys x 32 heads of block hb) by transpose reads of the [key][head] tile;
      // keys beyond the route hold the last slot's values, so zero them
      bf16x8 dso[2][2];                                     // [part hi/lo][head block]
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const char* sp = sb + pt * kSB;
          const int hc = 32 * hb + 16 * (g & 1) + 4 * (s16 & 3);
          const v4s x0 = lds_read_tr(reinterpret_cast<const uint16_t*>(sp + vr * 128 + 16 * ((hc >> 3) ^ (vr & 7)) + 2 * (hc & 7)));
          const v4s x1 = lds_read_tr(reinterpret_cast<const uint16_t*>(sp + (vr + 4) * 128 + 16 * ((hc >> 3) ^ ((vr + 4) & 7)) + 2 * (hc & 7)));
          dso[pt][hb] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          const int e0 = kKC * i + 8 * h32;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (e0 + j >= n) dso[pt][hb][j] = 0;
        }
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        if (k < ntw) {
          const int dcol = 32 * (wid + 4 * k) + 16 * (g & 1) + 4 * (s16 & 3);
          const v4s v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb + swz(vr, dcol)));
          const v4s v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb + swz(vr + 4, dcol)));
          const bf16x8 kt = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            acc[k][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dso[0][hb], acc[k][hb], 0, 0, 0);
            acc[k][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dso[1][hb], acc[k][hb], 0, 0, 0);
          }
        }
      }
    }
  }
  // dq rows: lane holds dims 32 tile + 8 q4 + 4 h32 + {0..3} of head 32 hb + l32
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    if (k >= ntw) continue;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      uint16_t* op = dq + (row * a.Hq + h0 + 32 * hb + l32) * kLD + 32 * (wid + 4 * k) + 4 * h32;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 u;
        u.x = pack_bf16x2(acc[k][hb][4 * q4] * a.scale, acc[k][hb][4 * q4 + 1] * a.scale);
        u.y = pack_bf16x2(acc[k][hb][4 * q4 + 2] * a.scale, acc[k][hb][4 * q4 + 3] * a.scale);
        *reinterpret_cast<uint2*>(op + 8 * q4) = u;
      }
    }
  }
}

// ---- dkv: per query, dKV[key, :] += scale dS^T q + [P^T dO, 0] into the FP32 accumulator
// wave w owns 16-dim tiles w, w + 4, ... of the 36 (dK) and of the 32 (dV)
__global__ void __launch_bounds__(256, 2)
latent_dkv_kernel(AttnArgs a, const uint16_t* __restrict__ pds, const uint16_t* __restrict__ qt,
                  const uint16_t* __restrict__ dot, float* __restrict__ dkv, int n_items) {
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const QItem it = decode_qitem(item, a.B, a.S_q, a.Hkv, 0);
  const int b = it.b, t = it.t, kvh = it.kvh;
  const int64_t row = static_cast<int64_t>(b) * a.S_q + t;
  const int64_t rrow = route_row(a, b, t, kvh);
  const int n = max(0, min(a.lens[rrow], a.L));
  if (n == 0) return;
  const int32_t* route = a.routes + rrow * a.L;
  const int64_t prow = row * a.Hkv + kvh;
  // B operands: k = heads 32 ks + 8 g16 .. + 8, column = dim 16 tile + l16
  constexpr int NK = kLD / 16 / 4, NV = kLDV / 16 / 4;      // 9 dK tiles, 8 dV tiles per wave
  bf16x8 bq[NK][2], bd[NV][2];
  {
    const uint16_t* qp = qt + (prow * kLD + 16 * wid + l16) * kHeads + 8 * g16;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bq[k][ks] = *reinterpret_cast<const bf16x8*>(qp + (64 * k) * kHeads + 32 * ks);
    const uint16_t* dp = dot + (prow * kLDV + 16 * wid + l16) * kHeads + 8 * g16;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bd[k][ks] = *reinterpret_cast<const bf16x8*>(dp + (64 * k) * kHeads + 32 * ks);
  }
  float* dbase = dkv + (static_cast<int64_t>(b) * a.S_k * a.Hkv + kvh) * kLD;
  const int64_t kstride = static_cast<int64_t>(a.Hkv) * kLD;
  const int nch = (n + kKC - 1) / kKC;
  // A operands of chunk ch: row = route slot 16 ch + l16, k = heads 32 ks + 8 g16 ..;
  // [0] the high, [1] the low bf16 parts
  struct Ops { bf16x8 p[2][2], d[2][2]; int id[4]; };
  auto load = [&](int ch, Ops& o) __attribute__((always_inline)) {
    const int e = min(kKC * ch + l16, n - 1);
    const uint16_t* src = pds + pds_row(prow, a.L, e) + 8 * g16;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        o.p[pt][ks] = *reinterpret_cast<const bf16x8*>(src + pt * kHeads + 32 * ks);
        o.d[pt][ks] = *reinterpret_cast<const bf16x8*>(src + 2 * kHeads + pt * kHeads + 32 * ks);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ej = kKC * ch + 4 * g16 + j;
      o.id[j] = ej < n ? route[ej] : -1;
    }
  };
  Ops cur;
  load(0, cur);
  for (int ch = 0; ch < nch; ++ch) {
    Ops nxt;
    if (ch + 1 < nch) load(ch + 1, nxt);
    // slots past the route repeat its last slot: their A rows are zeroed
    if (kKC * ch + l16 >= n) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          cur.p[pt][ks] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
          cur.d[pt][ks] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.d[pt][ks], bq[k][ks], acc, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] *= a.scale;
      if (k < NV) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.p[pt][ks], bd[k][ks], acc, 0, 0, 0);
      }
      const int dim = 16 * (wid + 4 * k) + l16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int id = cur.id[j];
        if (id >= 0 && id < a.S_k) unsafeAtomicAdd(dbase + id * kstride + dim, acc[j]);
      }
    }
    if (ch + 1 < nch) cur = nxt;
  }
}

__global__ void __launch_bounds__(256)
latent_final_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4*>(src + i);
  uint2 u;
  u.x = pack_bf16x2(v.x, v.y);
  u.y = pack_bf16x2(v.z, v.w);
  *reinterpret_cast<uint2*>(dst + i) = u;
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

size_t latent_bwd_workspace_bytes(int B, int S_q, int S_k, int L, int Hq, int Hkv) {
  const size_t rows = static_cast<size_t>(B) * S_q;
  const size_t rk = rows * Hkv;
  return al256(rows * Hq * 4) + al256(rk * kLD * kHeads * 2) + al256(rk * kLDV * kHeads * 2) +
         al256(rk * static_cast<size_t>(L) * kPdsW * 2) + al256(static_cast<size_t>(B) * S_k * Hkv * kLD * 4);
}

bool latent_bwd_applies(const AttnArgs& a, const void* dk, const void* dv) {
  const bool latent = a.v == a.k && a.sv_b == a.sk_b && a.sv_t == a.sk_t && a.sv_h == a.sk_h;
  // LDS of the ds pass (the largest): three chunk buffers, two P / dS tiles, the route
  const size_t ds_lds = 3 * static_cast<size_t>(kBufB) + 2 * kKC * kPdsW * 2 + static_cast<size_t>(a.L) * 4;
  return a.dtype == IRB_BF16 && a.Dqk == kLD && a.Dv == kLDV && latent && a.Hq == kHeads * a.Hkv && dk == dv &&
         ds_lds <= 150 * 1024;
}

int launch_latent_bwd(const AttnArgs& a, const void* dout, const float* lse, const float* out32, void* dq,
                      void* dkv_out, void* ws, int64_t* dropped, hipStream_t stream) {
  constexpr int NB = 3;
  const size_t rows = static_cast<size_t>(a.B) * a.S_q;
  const size_t rk = rows * a.Hkv;
  char* p = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(p);
  p += al256(rows * a.Hq * 4);
  uint16_t* qt = reinterpret_cast<uint16_t*>(p);
  p += al256(rk * kLD * kHeads * 2);
  uint16_t* dot = reinterpret_cast<uint16_t*>(p);
  p += al256(rk * kLDV * kHeads * 2);
  uint16_t* pds = reinterpret_cast<uint16_t*>(p);
  p += al256(rk * static_cast<size_t>(a.L) * kPdsW * 2);
  float* acc = reinterpret_cast<float*>(p);
  const int64_t nacc = static_cast<int64_t>(a.B) * a.S_k * a.Hkv * kLD;
  if (dropped)
    if (int rc = launch_fill_i32(reinterpret_cast<int32_t*>(dropped), 2, 0, stream)) return rc;
  if (int rc = launch_fill_i32(reinterpret_cast<int32_t*>(acc), nacc, 0, stream)) return rc;
  if (rk == 0) return 0;
  if (rk > 0x7fffffff) return static_cast<int>(hipErrorInvalidValue);
  const int items = static_cast<int>(rk);
  // Delta from the forward's FP32 output when given, else the forward again in Delta mode
  if (out32) {
    if (int rc = launch_delta_from_o(a, dout, out32, delta, stream)) return rc;
  } else if (int rc = launch_latent_fwd(a, nullptr, nullptr, dout, delta, true, stream)) {
    return rc;
  }
  hipLaunchKernelGGL(latent_prep_kernel, dim3(static_cast<unsigned>(rk), kLD / 64 + kLDV / 64), dim3(256), 0, stream, a,
                     static_cast<const uint16_t*>(dout), qt, dot);
  {
    const size_t lds = static_cast<size_t>(NB) * kBufB + 2 * kKC * kPdsW * 2 + static_cast<size_t>(a.L) * 4;
    auto kern = latent_ds_kernel<NB>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(items)), dim3(256), lds, stream, a,
                       static_cast<const uint16_t*>(dout), lse, delta, pds, items);
  }
  {
    const size_t lds = static_cast<size_t>(NB) * (kBufB + 2 * kKC * kHeads * 2) + static_cast<size_t>(a.L) * 4;
    auto kern = latent_dq_kernel<NB>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(items)), dim3(256), lds, stream, a,
                       static_cast<const uint16_t*>(pds), static_cast<uint16_t*>(dq), items);
  }
  hipLaunchKernelGGL(latent_dkv_kernel, dim3(static_cast<unsigned>(items)), dim3(256), 0, stream, a,
                     static_cast<const uint16_t*>(pds), static_cast<const uint16_t*>(qt),
                     static_cast<const uint16_t*>(dot), acc, items);
  hipLaunchKernelGGL(latent_final_kernel, dim3(static_cast<unsigned>((nacc / 4 + 255) / 256)), dim3(256), 0, stream,
                     acc, static_cast<uint16_t*>(dkv_out), nacc);
  return 0;
}

// bf16 latent rows (Dqk 576, Dv 512, value = the key row's first 512
// channels) with 64 query heads per KV head.  Returns -1 when the shape is not
// this kernel's (the caller then uses the general path).
static int latent_nb() {
  static int v = [] {
    const char* e = getenv("IRB_LATENT_NB");
    const int x = e ? atoi(e) : 3;
    return (x == 3 || x == 4) ? x : 3;
  }();
  return v;
}

int launch_latent_fwd(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, bool delta_mode,
                      hipStream_t stream) {
  const bool latent = a.v == a.k && a.sv_b == a.sk_b && a.sv_t == a.sk_t && a.sv_h == a.sk_h;
  if (a.dtype != IRB_BF16 || a.Dqk != kLD || a.Dv != kLDV || !latent || a.Hq != kHeads * a.Hkv) return -1;
  const int NB = latent_nb();
  const size_t lds = latent_fwd_lds(NB, a.L);
  if (lds > 150 * 1024) return -1;
  const int64_t items = static_cast<int64_t>(a.B) * a.S_q * a.Hkv;
  if (items == 0) return 0;
  if (items > 0x7fffffff) return -1;
  using K = void (*)(AttnArgs, uint16_t*, float*, const uint16_t*, float*, int);
  const K kern = NB == 4 ? (delta_mode ? latent_fwd_kernel<4, true> : latent_fwd_kernel<4, false>)
                         : (delta_mode ? latent_fwd_kernel<3, true> : latent_fwd_kernel<3, false>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return static_cast<int>(e);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(items)), dim3(256), lds, stream, a,
                     static_cast<uint16_t*>(out), lse, static_cast<const uint16_t*>(dout), delta,
                     static_cast<int>(items));
  return 0;
}

}  // namespace irb
