// Launcher prototypes shared by the kernel translation units and the C ABI.
// Launchers assume validated arguments (see abi.hip) and return 0 or a HIP error code.
#pragma once

#include "../../include/irb.h"
#include "irb_common.hpp"

namespace irb {

int launch_compress(const Layout& L, int c, const void* k, int dtype, int64_t sb, int64_t st, int D,
                    const float* gamma, float eps, const float* freqs, int R, float* kc,
                    int32_t* cu_blocks, hipStream_t stream);

// normalised, rotated index queries: n_rows = tokens * H rows of D contiguous
// elements; rope rows [tokens, R]; out may alias q
int launch_prep_queries(const void* q, int dtype, int64_t n_rows, int H, int D, const float* gamma, float eps,
                        const float* rope, int R, void* out, hipStream_t stream);

// write_invisible: also write -inf at the tile's invisible entries (the fused
// route path skips them: selection never reads them); queries with at most
// skip_nb visible blocks are not scored (-1: score every query)
// kc_split (optional): the keys pre-split by launch_split_keys, streamed by
// direct global-to-LDS loads instead of being split while staging.
// n_grp: index queries [B, S, n_grp, H, D] and weights [B, S, n_grp, H] with
// q and w pointing at one group's heads (1: [B, S, H, D] and [B, S, H])
// Index-query preparation applied by the score kernel as it loads raw
// queries (gamma == nullptr: the queries are used as they are).  Same
// arithmetic as launch_prep_queries, so the scores equal those of prepared
// queries; needs R == 0 or R a multiple of 64 up to D (each lane then holds
// the rotation partners of its own dimensions).
struct QPrep {
  const float* gamma = nullptr;
  const float* rope = nullptr;   // [B * S, R] rotary rows
  float eps = 0.f;
  int R = 0;
};
bool score_prep_ok(int D, int R);
int launch_score_tile(const Layout& L, const void* q, int dtype, int H, int D, const float* w,
                      const float* kc, const uint16_t* kc_split, const int32_t* cu_blocks, int c, float scale,
                      int q0, int q1, int j0, int j1, float* out, int64_t out_stride, int write_invisible,
                      int skip_nb, int n_grp, hipStream_t stream, const QPrep& prep = QPrep{});
// All groups of 4 or 8 heads in one launch (bf16 queries [B, S, groups,
// H_group, D], weights [B, S, groups, H_group], groups * H_group in {16, 32},
// D in {64, 128}): group g's tile at out + g * group_stride, each laid out as
// launch_score_tile's.
bool score_grouped_ok(int dtype, int groups, int H_group, int D);
int launch_score_grouped(const Layout& L, const void* q, int dtype, int groups, int H_group, int D, const float* w,
                         const float* kc, const uint16_t* kc_split, const int32_t* cu_blocks, int c, float scale,
                         int q0, int q1, int j0, int j1, float* out, int64_t out_stride, int64_t group_stride,
                         int write_invisible, int skip_nb, hipStream_t stream);
// kcs[2 blk] = bf16 high halves of kc[blk], kcs[2 blk + 1] = low halves (rows of D)
int launch_split_keys(const float* kc, uint16_t* kcs, int64_t n_blocks, int D, hipStream_t stream);

// hist_only = 1: a query sees only the complete blocks before its own group's
// block (floor(pos / c) of them: the CSA historical regions), else floor((pos + 1) / c)
int launch_select(const Layout& L, const float* scores, int64_t stride, int q0, int q1,
                  const int32_t* cu_blocks, int c, int topk, int32_t* sel, int32_t* cnt,
                  hipStream_t stream, int hist_only = 0);

// CSA variant (csa.hip)
int launch_round_e4m3(const void* x, int dtype, int64_t n, uint16_t* out, hipStream_t stream);
int launch_gather_payload(const void* keys, const void* logits, int esize, int B, int T, int D, const int32_t* sources,
                          const uint8_t* valid, int R, int rs, void* pk, void* pz, hipStream_t stream);
int launch_summarize(const void* pk, const void* pz, int dtype, const uint8_t* valid, int B, int R, int rs, int D,
                     uint16_t* summary, hipStream_t stream);
size_t region_ids_workspace_bytes(int B, int S, int topk, int num_docs);
int launch_region_ids(const Layout& L, const float* scores, int64_t stride, int q0, int q1, const int32_t* cu_blocks,
                      int c, int topk, int32_t* ids, int32_t* cnt, void* ws, hipStream_t stream);

int launch_expand(const Layout& L, const int32_t* sel, const int32_t* cnt, int topk, int c, int window,
                  const int32_t* cu_blocks, int Lw, int32_t* routes, int32_t* lens, hipStream_t stream);

int launch_compact(const int32_t* in, int64_t rows, int width, int64_t key_count, int32_t* out,
                   int32_t* lens, int32_t* bad, hipStream_t stream);

// key-membership words [rows, ceil(keys / 32)] of the first lens[row] entries of route rows [rows, L]; keys <= 131072
int launch_route_bits(const int32_t* routes, const int32_t* lens, int64_t rows, int L, int keys, uint32_t* bits,
                      hipStream_t stream);
// membership words [rows, ceil(regions / 32)] of id rows [rows, slots]; regions <= 131072
int launch_bitmap(const int32_t* ids, int64_t rows, int slots, int regions, int32_t* bitmap, hipStream_t stream);

// full/partial split of a block list (lists as written by launch_block_lists);
// cover (split_cover_bytes, one-query tiles only, else nullptr): scratch for
// the per-(query, key tile) coverage bits
size_t split_cover_bytes(int B, int S_q, int S_k, int bq, int bk);
int launch_split_full_blocks(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int Lw, int bq,
                             int bk, int reverse, const int32_t* counts, const int32_t* indices, int width,
                             int32_t* full_counts, int32_t* full_indices, int32_t* part_counts,
                             int32_t* part_indices, uint32_t* cover, hipStream_t stream);
int launch_block_lists(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int Lw,
                       int bq, int bk, int reverse, int32_t* counts, int32_t* indices, int width,
                       uint32_t* bitmap, hipStream_t stream);

struct AttnArgs {
  const void* q; const void* k; const void* v;
  int64_t sq_b, sq_t, sq_h, sk_b, sk_t, sk_h, sv_b, sv_t, sv_h;
  const int32_t* routes; const int32_t* lens;
  int B, S_q, S_k, L, Hq, Hkv, Dqk, Dv;
  float scale;
  int dtype;
  int RG;   // route groups: 1 (one route per query, every head) or Hkv (one per KV group)
  float* o32;   // forward, nullable: o also in FP32, [B, S_q, Hq, Dv] (the backward's Delta input)
};

// Row of (batch b, query t) in the routes / lens read by KV head kvh.  Routes
// are laid out group-major, [RG, B, S_q, L]: with RG = Hkv each KV group has
// its own route per query (the CSA page's per-group selections), with RG = 1
// all heads share it.
__device__ __forceinline__ int64_t route_row(const AttnArgs& a, int b, int t, int kvh) {
  return (static_cast<int64_t>(a.RG > 1 ? kvh : 0) * a.B + b) * a.S_q + t;
}

// ---- query tiles (forward and dq query-tile kernels)
constexpr int kSegTiles = 256;   // 32-key tiles per mask segment (8192 keys)

// route-density threshold (per mille) above which a query tile runs on the
// query-tile kernels (IRB_TILE_MIN_DENSITY overrides it)
int tile_thr_milli();

// Statistics of the query tile [qa, qa + BQ) of batch b, KV head kvh: whether
// its routes are dense enough in their key range for the tile kernels.
struct TileStats {
  bool dense;
  int kmin, kmax;
  int n_lane, last_lane;   // lane q < BQ: route length of query qa + q and its last entry
};

// Evaluated by a whole wavefront (uniform result).  BQ <= 64.
__device__ __forceinline__ TileStats tile_stats_wave(const AttnArgs& a, int b, int kvh, int qa, int BQ, int thr_milli) {
  const int lane = threadIdx.x & 63;
  int kmin = 0x7fffffff, kmax = -1, total = 0, valid = 0;
  const int t = qa + lane;
  if (lane < BQ && t < a.S_q) {
    const int64_t rrow = route_row(a, b, t, kvh);
    const int n = max(0, min(a.lens[rrow], a.L));
    valid = 1;
    if (n > 0) {
      const int32_t* r = a.routes + rrow * a.L;
      kmin = r[0];
      kmax = r[n - 1];
      total = n;
    }
  }
  const int lane_n = total, lane_last = kmax;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, __shfl_xor(kmin, o, 64));
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    total += __shfl_xor(total, o, 64);
    valid += __shfl_xor(valid, o, 64);
  }
  TileStats st;
  st.kmin = max(kmin, 0);
  st.kmax = min(kmax, a.S_k - 1);
  const int64_t span = st.kmax >= st.kmin ? static_cast<int64_t>(st.kmax - st.kmin + 1) : 0;
  st.dense = total > 0 && span > 0 && static_cast<int64_t>(total) * 1000 >= static_cast<int64_t>(thr_milli) * valid * span;
  st.n_lane = lane_n;
  st.last_lane = lane_last;
  return st;
}


// Per-query gather kernels visit work items (b, t, KV head).  When the K/V rows
// of all heads outgrow the chip's last-level cache (256 MiB of Infinity Cache
// on MI355X; half of it is the threshold), the items run head-major -- every
// query of one KV head before the next head -- so the rows the running
// wavefronts gather stay cache-resident; otherwise the heads of one query run
// side by side (measured faster when everything fits).
inline bool gather_head_major(const AttnArgs& a) {
  const int64_t elem = a.dtype == IRB_BF16 ? 2 : 4;
  const int64_t kv_bytes = static_cast<int64_t>(a.B) * a.S_k * a.Hkv * (a.Dqk + a.Dv) * elem;
  return kv_bytes > (int64_t{128} << 20);
}

// ws (nullable): at least attn_fwd_qbits_bytes(a) bytes for the per-route-row
// key-membership words of the query-tile kernel (else its masks come from the routes)
size_t attn_fwd_qbits_bytes(const AttnArgs& a);
int launch_attn_fwd(const AttnArgs& a, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);
// bf16 shared latent rows (576 / 512) with 64 heads per KV head: o and lse, or
// (delta_mode) Delta[b,h,t] = rowsum(dO * o) with o in FP32; -1 if the shape is not its own
int launch_latent_fwd(const AttnArgs& a, void* out, float* lse, const void* dout, float* delta, bool delta_mode,
                      hipStream_t stream);
// query-major latent backward (bf16 576 / 512 with v aliasing k, 64 heads per
// KV head, merged dk == dv): its workspace bytes, whether it applies, and the launch
size_t latent_bwd_workspace_bytes(int B, int S_q, int S_k, int L, int Hq, int Hkv);
bool latent_bwd_applies(const AttnArgs& a, const void* dk, const void* dv);
int launch_latent_bwd(const AttnArgs& a, const void* dout, const float* lse, const float* out32, void* dq,
                      void* dkv_out, void* ws, int64_t* dropped, hipStream_t stream);
// Delta[b,h,t] = rowsum(dO * o) from the forward's FP32 o
int launch_delta_from_o(const AttnArgs& a, const void* dout, const float* o32, float* delta, hipStream_t stream);
// backward row statistic Delta[b,h,t] = rowsum(dO * o) with o recomputed in FP32
int launch_attn_delta(const AttnArgs& a, const void* dout, float* delta, hipStream_t stream);

struct AttnBwdArgs {
  AttnArgs f;
  const float* out32;   // nullable: the forward's FP32 o; Delta = rowsum(dO * o) is then read off it
  const void* dout; const float* lse;
  const int32_t* rev_counts; const int32_t* rev_indices;
  int rev_bq, rev_bk, rev_width;
  void* dq; void* dk; void* dv;
  void* ws; size_t ws_bytes;
  int64_t* dropped;   // device, nullable: receives the hits past the workspace's capacity
};

size_t attn_bwd_workspace_bytes(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv, int dtype,
                                int RG);
int launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);
bool attn_bwd_reads_out32(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv, int dtype, int RG);

// fill a device int32 range with a value (a kernel, so callers may capture it in graphs)
int launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);

}  // namespace irb
