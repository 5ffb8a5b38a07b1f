// C ABI of libirb: argument validation, error reporting and dispatch.
// Every entry point validates on the host, enqueues on the caller's stream and
// returns without synchronising.  See include/irb.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "irb_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return IRB_OK;
}

// 1 if the current device is a gfx950, cached per device
int device_ok() {
  static int cache[64];   // 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    cache[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  return cache[dev] == 1;
}

#define IRB_REQUIRE_DEVICE()                                                                  \
  do {                                                                                        \
    if (!device_ok()) return fail(IRB_ERR_UNAVAILABLE, "%s: no gfx950 device is current", __func__); \
  } while (0)

int launched(const char* fn, int rc) {
  hipError_t e = rc ? static_cast<hipError_t>(rc) : hipGetLastError();
  if (e != hipSuccess) return fail(IRB_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

int check_layout(const char* fn, const irb_layout* L, irb::Layout& out) {
  if (!L) return fail(IRB_ERR_INVALID, "%s: layout is NULL", fn);
  if (L->B < 1 || L->S < 1) return fail(IRB_ERR_INVALID, "%s: layout needs B >= 1 and S >= 1 (got %d, %d)", fn, L->B, L->S);
  if (L->cu_seqlens && L->row_lens) return fail(IRB_ERR_INVALID, "%s: give cu_seqlens or row_lens, not both", fn);
  if (L->cu_seqlens && L->B != 1) return fail(IRB_ERR_INVALID, "%s: packed documents need B == 1", fn);
  if (L->cu_seqlens && L->num_docs < 1) return fail(IRB_ERR_INVALID, "%s: packed layout needs num_docs >= 1", fn);
  out.B = L->B;
  out.S = L->S;
  out.cu_seqlens = L->cu_seqlens;
  out.num_docs = L->cu_seqlens ? L->num_docs : 0;
  out.row_lens = L->row_lens;
  return 0;
}

int check_dtype(const char* fn, int dtype) {
  if (dtype != IRB_F32 && dtype != IRB_BF16) return fail(IRB_ERR_DTYPE, "%s: dtype must be IRB_F32 or IRB_BF16 (got %d)", fn, dtype);
  return 0;
}

bool score_heads_ok(int H) { return H >= 4 && H <= 64 && H % 4 == 0 && (16 % H == 0 || H % 16 == 0); }

// Scratch of irb_route_topk_fused_noalloc: one copy per GPU the library runs
// on, held until the process ends.  Host code never passes `scratch` itself
// (in host code the name is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept in g_scratch_dev.
std::mutex g_scratch_mu;
void* g_scratch_dev[64];

}  // namespace

static __device__ __align__(256) unsigned char scratch[IRB_NOALLOC_SCRATCH_BYTES];

namespace {

// device address of this device's scratch (looked up on the first call on the device)
int scratch_ptr(const char* fn, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(IRB_ERR_HIP, "%s: no current device", fn);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(IRB_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return 0;
}

}  // namespace

extern "C" {

int irb_is_available(void) { return device_ok(); }

const char* irb_last_error(void) { return g_err.c_str(); }

const char* irb_version(void) { return "irb 0.1.0 gfx950"; }

int irb_compress_keys(const irb_layout* layout, int c, const void* k_idx, int dtype, int64_t stride_b,
                      int64_t stride_t, int D_idx, const float* gamma, float eps, const float* freqs, int D_rope,
                      float* kc, int32_t* cu_blocks, void* stream) {
  const char* fn = "irb_compress_keys";
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (int r = check_dtype(fn, dtype)) return r;
  if (c < 1 || c > 64) return fail(IRB_ERR_INVALID, "%s: c must be in 1..64 (got %d)", fn, c);
  if (D_idx < 32 || D_idx > 512 || D_idx % 32) return fail(IRB_ERR_INVALID, "%s: D_idx must be a multiple of 32 in 32..512", fn);
  if (D_rope < 0 || D_rope > D_idx || D_rope % 2) return fail(IRB_ERR_INVALID, "%s: D_rope must be even and <= D_idx", fn);
  if (stride_t < D_idx || stride_b < 0) return fail(IRB_ERR_INVALID, "%s: bad k_idx strides", fn);
  if (!k_idx || !gamma || !kc || (D_rope > 0 && !freqs)) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks output", fn);
  if (!(eps >= 0.f)) return fail(IRB_ERR_INVALID, "%s: eps must be >= 0", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_compress(L, c, k_idx, dtype, stride_b, stride_t, D_idx, gamma, eps, freqs, D_rope, kc,
                                           cu_blocks, static_cast<hipStream_t>(stream)));
}

int irb_prepare_index_queries(const void* q_raw, int dtype, int64_t n_tokens, int H_idx, int D_idx,
                              const float* gamma, float eps, const float* rope, int D_rope, void* q_out,
                              void* stream) {
  const char* fn = "irb_prepare_index_queries";
  if (int r = check_dtype(fn, dtype)) return r;
  if (n_tokens < 0 || H_idx < 1 || n_tokens > (int64_t{1} << 40) / H_idx)
    return fail(IRB_ERR_INVALID, "%s: need n_tokens >= 0 and H_idx >= 1", fn);
  if (D_idx != 32 && D_idx != 64 && D_idx != 128 && D_idx != 256 && D_idx != 512)
    return fail(IRB_ERR_INVALID, "%s: D_idx must be 32, 64, 128, 256 or 512 (got %d)", fn, D_idx);
  if (D_rope < 0 || D_rope > D_idx || D_rope % 2) return fail(IRB_ERR_INVALID, "%s: D_rope must be even and <= D_idx", fn);
  if (!q_raw || !gamma || !q_out || (D_rope > 0 && !rope)) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if ((reinterpret_cast<uintptr_t>(q_raw) | reinterpret_cast<uintptr_t>(q_out)) & 15)
    return fail(IRB_ERR_INVALID, "%s: q_raw and q_out must be 16-byte aligned", fn);
  if (!(eps >= 0.f)) return fail(IRB_ERR_INVALID, "%s: eps must be >= 0", fn);
  if (n_tokens == 0) return 0;
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_prep_queries(q_raw, dtype, n_tokens * H_idx, H_idx, D_idx, gamma, eps, rope, D_rope,
                                               q_out, static_cast<hipStream_t>(stream)));
}

// groups >= 1 index-query groups per token; group g's tile lands at
// out + g * B * (q1 - q0) * out_row_stride
static int score_tile_impl(const char* fn, const irb_layout* layout, const void* q_idx, int dtype, int groups,
                           int H_idx, int D_idx, const float* w, const float* kc, const int32_t* cu_blocks, int c,
                           float score_scale, int q0, int q1, int j0, int j1, float* out, int64_t out_row_stride,
                           void* stream) {
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (int r = check_dtype(fn, dtype)) return r;
  if (!score_heads_ok(H_idx)) return fail(IRB_ERR_INVALID, "%s: H_idx must be 4, 8, 16 or a multiple of 16 up to 64 (got %d)", fn, H_idx);
  if (D_idx != 32 && D_idx != 64 && D_idx != 128) return fail(IRB_ERR_INVALID, "%s: D_idx must be 32, 64 or 128 (got %d)", fn, D_idx);
  if (c < 1) return fail(IRB_ERR_INVALID, "%s: c must be >= 1", fn);
  if (score_scale == 0.f) score_scale = 1.f / std::sqrt(static_cast<float>(D_idx));
  if (!(score_scale > 0.f) || !std::isfinite(score_scale))
    return fail(IRB_ERR_INVALID, "%s: score_scale must be finite and > 0 (0 = 1/sqrt(D_idx))", fn);
  if (q0 < 0 || q1 <= q0 || q1 > L.S) return fail(IRB_ERR_INVALID, "%s: need 0 <= q0 < q1 <= S", fn);
  if (j0 < 0 || j1 <= j0 || j1 > L.S / c) return fail(IRB_ERR_INVALID, "%s: need 0 <= j0 < j1 <= S/c", fn);
  if (out_row_stride < j1 - j0) return fail(IRB_ERR_INVALID, "%s: out_row_stride < j1 - j0", fn);
  if (!q_idx || !w || !kc || !out) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks", fn);
  if (groups < 1 || groups > 64) return fail(IRB_ERR_INVALID, "%s: groups must be in 1..64 (got %d)", fn, groups);
  IRB_REQUIRE_DEVICE();
  const int esz = dtype == IRB_BF16 ? 2 : 4;
  const int64_t tile = static_cast<int64_t>(L.B) * (q1 - q0) * out_row_stride;
  if (groups > 1 && irb::score_grouped_ok(dtype, groups, H_idx, D_idx))
    return launched(fn, irb::launch_score_grouped(L, q_idx, dtype, groups, H_idx, D_idx, w, kc, nullptr, cu_blocks, c,
                                                  score_scale, q0, q1, j0, j1, out, out_row_stride, tile, 1, -1,
                                                  static_cast<hipStream_t>(stream)));
  for (int g = 0; g < groups; ++g) {
    const void* qg = static_cast<const char*>(q_idx) + static_cast<int64_t>(g) * H_idx * D_idx * esz;
    const int rc = irb::launch_score_tile(L, qg, dtype, H_idx, D_idx, w + static_cast<int64_t>(g) * H_idx, kc, nullptr,
                                          cu_blocks, c, score_scale, q0, q1, j0, j1, out + g * tile, out_row_stride, 1,
                                          -1, groups, static_cast<hipStream_t>(stream));
    if (rc) return launched(fn, rc);
  }
  return launched(fn, 0);
}

int irb_indexer_score_tile(const irb_layout* layout, const void* q_idx, int dtype, int H_idx, int D_idx,
                           const float* w, const float* kc, const int32_t* cu_blocks, int c, float score_scale,
                           int q0, int q1, int j0, int j1, float* out, int64_t out_row_stride, void* stream) {
  return score_tile_impl("irb_indexer_score_tile", layout, q_idx, dtype, 1, H_idx, D_idx, w, kc, cu_blocks, c,
                         score_scale, q0, q1, j0, j1, out, out_row_stride, stream);
}

int irb_indexer_score_tile_groups(const irb_layout* layout, const void* q_idx, int dtype, int groups, int H_idx,
                                  int D_idx, const float* w, const float* kc, const int32_t* cu_blocks, int c,
                                  float score_scale, int q0, int q1, int j0, int j1, float* out,
                                  int64_t out_row_stride, void* stream) {
  return score_tile_impl("irb_indexer_score_tile_groups", layout, q_idx, dtype, groups, H_idx, D_idx, w, kc,
                         cu_blocks, c, score_scale, q0, q1, j0, j1, out, out_row_stride, stream);
}

int irb_select_topk_regions(const irb_layout* layout, const float* scores, int64_t score_row_stride, int q0, int q1,
                            const int32_t* cu_blocks, int c, int topk, int32_t* sel, int32_t* cnt, void* stream) {
  const char* fn = "irb_select_topk_regions";
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (c < 1) return fail(IRB_ERR_INVALID, "%s: c must be >= 1", fn);
  if (topk < 1 || topk > 4096) return fail(IRB_ERR_INVALID, "%s: topk must be in 1..4096 (got %d)", fn, topk);
  if (q0 < 0 || q1 <= q0 || q1 > L.S) return fail(IRB_ERR_INVALID, "%s: need 0 <= q0 < q1 <= S", fn);
  if (score_row_stride < 1) return fail(IRB_ERR_INVALID, "%s: score_row_stride must be >= 1", fn);
  if (!scores || !sel || !cnt) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_select(L, scores, score_row_stride, q0, q1, cu_blocks, c, topk, sel, cnt,
                                         static_cast<hipStream_t>(stream)));
}

// fused-route workspace: the keys split into bf16 high/low rows, then score rows
static size_t split_keys_bytes(int B, int nb, int D_idx) {
  return (static_cast<size_t>(B) * std::max(nb, 0) * D_idx * 4 + 255) / 256 * 256;
}

size_t irb_route_topk_fused_workspace_size(int B, int S, int c, int D_idx, int topk, int q0, int q1) {
  (void)topk;
  if (B < 1 || S < 1 || c < 1 || q1 <= q0) return 0;
  if (D_idx != 32 && D_idx != 64 && D_idx != 128) return 0;
  const int64_t nb = S / c;
  const int64_t rows_budget = nb > 0 ? ((static_cast<int64_t>(256) << 20) / (4 * nb)) : 1;
  const int64_t rows = std::min<int64_t>(std::max<int64_t>(rows_budget / B, 512), q1 - q0);
  return split_keys_bytes(B, static_cast<int>(nb), D_idx) + static_cast<size_t>(rows * B * std::max<int64_t>(nb, 1) * 4);
}

size_t irb_route_topk_fused_groups_workspace_size(int B, int S, int c, int D_idx, int topk, int q0, int q1,
                                                  int groups) {
  if (groups < 1 || groups > 64) return 0;
  const size_t one = irb_route_topk_fused_workspace_size(B, S, c, D_idx, topk, q0, q1);
  if (one == 0) return 0;
  const int nb = S / c;
  const size_t kbytes = split_keys_bytes(B, nb, D_idx);
  return kbytes + static_cast<size_t>(groups) * (one - kbytes);
}

// groups >= 1 index-query groups per token: group g selects into
// sel + g * B * S * topk and cnt + g * B * S; the split keys serve every group
static int route_fused_impl(const char* fn, const irb_layout* layout, const void* q_idx, int dtype, int groups,
                            int H_idx, int D_idx, const float* w, const float* kc, const int32_t* cu_blocks, int c,
                            float score_scale, int topk, int q0, int q1, int32_t* sel, int32_t* cnt, void* workspace,
                            size_t ws_bytes, void* stream, bool static_scratch = false,
                            const irb::QPrep& prep = irb::QPrep{}) {
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (int r = check_dtype(fn, dtype)) return r;
  if (!score_heads_ok(H_idx)) return fail(IRB_ERR_INVALID, "%s: unsupported H_idx %d", fn, H_idx);
  if (D_idx != 32 && D_idx != 64 && D_idx != 128) return fail(IRB_ERR_INVALID, "%s: D_idx must be 32, 64 or 128", fn);
  if (c < 1 || topk < 1 || topk > 4096) return fail(IRB_ERR_INVALID, "%s: bad c or topk", fn);
  if (score_scale == 0.f) score_scale = 1.f / std::sqrt(static_cast<float>(D_idx));
  if (!(score_scale > 0.f) || !std::isfinite(score_scale))
    return fail(IRB_ERR_INVALID, "%s: score_scale must be finite and > 0 (0 = 1/sqrt(D_idx))", fn);
  if (q0 < 0 || q1 <= q0 || q1 > L.S) return fail(IRB_ERR_INVALID, "%s: need 0 <= q0 < q1 <= S", fn);
  if (!q_idx || !w || !kc || !sel || !cnt || (!workspace && !static_scratch))
    return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks", fn);
  const int nb = L.S / c;
  if (nb < 1) return fail(IRB_ERR_INVALID, "%s: S/c must be >= 1", fn);
  if (groups < 1 || groups > 64) return fail(IRB_ERR_INVALID, "%s: groups must be in 1..64 (got %d)", fn, groups);
  // all groups scored by one launch (score tiles of every group alive at once), else group by group
  const bool one_launch = groups > 1 && irb::score_grouped_ok(dtype, groups, H_idx, D_idx);
  const int64_t per_row = static_cast<int64_t>(L.B) * nb * 4 * (one_launch ? groups : 1);
  const size_t kbytes = split_keys_bytes(L.B, nb, D_idx);
  if (static_scratch) {
    ws_bytes = IRB_NOALLOC_SCRATCH_BYTES;
    if (kbytes + static_cast<size_t>(per_row) > ws_bytes)
      return fail(IRB_ERR_INVALID,
                  "%s: B * (S/c) = %lld blocks of %d dims need %zu bytes of scratch (split keys and one score row); "
                  "the static maximum is %zu bytes",
                  fn, static_cast<long long>(L.B) * nb, D_idx, kbytes + static_cast<size_t>(per_row), ws_bytes);
  }
  const int64_t rows = ws_bytes > kbytes ? static_cast<int64_t>(ws_bytes - kbytes) / per_row : 0;
  if (rows < 1) return fail(IRB_ERR_INVALID, "%s: workspace too small (%zu bytes)", fn, ws_bytes);
  IRB_REQUIRE_DEVICE();
  if (static_scratch)
    if (int r = scratch_ptr(fn, &workspace)) return r;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* kcs = static_cast<uint16_t*>(workspace);
  float* scores = reinterpret_cast<float*>(static_cast<char*>(workspace) + kbytes);
  if (int rc = irb::launch_split_keys(kc, kcs, static_cast<int64_t>(L.B) * nb, D_idx, st)) return launched(fn, rc);
  const int esz = dtype == IRB_BF16 ? 2 : 4;
  const int64_t sel_group = static_cast<int64_t>(L.B) * L.S;
  if (one_launch) {
    for (int a = q0; a < q1; a += static_cast<int>(std::min<int64_t>(rows, q1 - a))) {
      const int e = a + static_cast<int>(std::min<int64_t>(rows, q1 - a));
      const int64_t gstride = static_cast<int64_t>(L.B) * (e - a) * nb;
      int rc = irb::launch_score_grouped(L, q_idx, dtype, groups, H_idx, D_idx, w, kc, kcs, cu_blocks, c, score_scale,
                                         a, e, 0, nb, scores, nb, gstride, 0, topk, st);
      for (int g = 0; g < groups && !rc; ++g)
        rc = irb::launch_select(L, scores + g * gstride, nb, a, e, cu_blocks, c, topk, sel + g * sel_group * topk,
                                cnt + g * sel_group, st);
      if (rc) return launched(fn, rc);
    }
    return launched(fn, 0);
  }
  for (int g = 0; g < groups; ++g) {
    const void* qg = static_cast<const char*>(q_idx) + static_cast<int64_t>(g) * H_idx * D_idx * esz;
    const float* wg = w + static_cast<int64_t>(g) * H_idx;
    for (int a = q0; a < q1; a += static_cast<int>(std::min<int64_t>(rows, q1 - a))) {
      const int e = a + static_cast<int>(std::min<int64_t>(rows, q1 - a));
      int rc = irb::launch_score_tile(L, qg, dtype, H_idx, D_idx, wg, kc, kcs, cu_blocks, c, score_scale, a, e, 0, nb,
                                      scores, nb, 0, topk, groups, st, prep);
      if (!rc)
        rc = irb::launch_select(L, scores, nb, a, e, cu_blocks, c, topk, sel + g * sel_group * topk,
                                cnt + g * sel_group, st);
      if (rc) return launched(fn, rc);
    }
  }
  return launched(fn, 0);
}

int irb_route_topk_fused(const irb_layout* layout, const void* q_idx, int dtype, int H_idx, int D_idx, const float* w,
                         const float* kc, const int32_t* cu_blocks, int c, float score_scale, int topk, int q0, int q1,
                         int32_t* sel, int32_t* cnt, void* workspace, size_t ws_bytes, void* stream) {
  return route_fused_impl("irb_route_topk_fused", layout, q_idx, dtype, 1, H_idx, D_idx, w, kc, cu_blocks, c,
                          score_scale, topk, q0, q1, sel, cnt, workspace, ws_bytes, stream);
}

int irb_route_topk_fused_raw(const irb_layout* layout, const void* q_raw, int dtype, int H_idx, int D_idx,
                             const float* gamma, float eps, const float* rope, int D_rope, const float* w,
                             const float* kc, const int32_t* cu_blocks, int c, float score_scale, int topk, int q0,
                             int q1, int32_t* sel, int32_t* cnt, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "irb_route_topk_fused_raw";
  if (!gamma || (reinterpret_cast<uintptr_t>(gamma) & 15)) return fail(IRB_ERR_INVALID, "%s: gamma must be a 16-byte aligned fp32 [D_idx] tensor", fn);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(IRB_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
  if (!irb::score_prep_ok(D_idx, D_rope))
    return fail(IRB_ERR_INVALID, "%s: D_rope must be 0 or a multiple of 64 up to D_idx (got %d, D_idx %d)", fn, D_rope, D_idx);
  if (D_rope > 0 && (!rope || (reinterpret_cast<uintptr_t>(rope) & 15)))
    return fail(IRB_ERR_INVALID, "%s: rope must be a 16-byte aligned fp32 [B, S, D_rope] tensor", fn);
  irb::QPrep prep;
  prep.gamma = gamma;
  prep.rope = D_rope > 0 ? rope : nullptr;
  prep.eps = eps;
  prep.R = D_rope;
  return route_fused_impl(fn, layout, q_raw, dtype, 1, H_idx, D_idx, w, kc, cu_blocks, c, score_scale, topk, q0, q1,
                          sel, cnt, workspace, ws_bytes, stream, false, prep);
}

int irb_route_topk_fused_noalloc(const irb_layout* layout, const void* q_idx, int dtype, int H_idx, int D_idx,
                                 const float* w, const float* kc, const int32_t* cu_blocks, int c, float score_scale,
                                 int topk, int q0, int q1, int32_t* sel, int32_t* cnt, void* stream) {
  return route_fused_impl("irb_route_topk_fused_noalloc", layout, q_idx, dtype, 1, H_idx, D_idx, w, kc, cu_blocks, c,
                          score_scale, topk, q0, q1, sel, cnt, nullptr, 0, stream, true);
}

int irb_route_topk_fused_groups(const irb_layout* layout, const void* q_idx, int dtype, int groups, int H_idx,
                                int D_idx, const float* w, const float* kc, const int32_t* cu_blocks, int c,
                                float score_scale, int topk, int q0, int q1, int32_t* sel, int32_t* cnt,
                                void* workspace, size_t ws_bytes, void* stream) {
  return route_fused_impl("irb_route_topk_fused_groups", layout, q_idx, dtype, groups, H_idx, D_idx, w, kc, cu_blocks,
                          c, score_scale, topk, q0, q1, sel, cnt, workspace, ws_bytes, stream);
}

int irb_round_e4m3(const void* x, int dtype, int64_t n, uint16_t* out, void* stream) {
  const char* fn = "irb_round_e4m3";
  if (int r = check_dtype(fn, dtype)) return r;
  if (n < 0) return fail(IRB_ERR_INVALID, "%s: n must be >= 0", fn);
  if (n == 0) return ok();
  if (!x || !out) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_round_e4m3(x, dtype, n, out, static_cast<hipStream_t>(stream)));
}

int irb_gather_region_payload(const void* keys, const void* logits, int dtype, int B, int T, int D,
                              const int32_t* sources, const uint8_t* valid, int R, int region_size, void* packed_keys,
                              void* packed_logits, void* stream) {
  const char* fn = "irb_gather_region_payload";
  if (int r = check_dtype(fn, dtype)) return r;
  const int esize = dtype == IRB_BF16 ? 2 : 4;
  if (B < 1 || T < 1 || D < 1 || R < 0 || region_size < 1) return fail(IRB_ERR_INVALID, "%s: bad sizes", fn);
  if ((D * esize) % 16) return fail(IRB_ERR_INVALID, "%s: D * element size must be a multiple of 16 bytes", fn);
  if (!keys || !logits || !sources || !packed_keys || !packed_logits) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if ((reinterpret_cast<uintptr_t>(keys) | reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(packed_keys) |
       reinterpret_cast<uintptr_t>(packed_logits)) & 15)
    return fail(IRB_ERR_INVALID, "%s: keys, logits and outputs must be 16-byte aligned", fn);
  if (R == 0) return ok();
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_gather_payload(keys, logits, esize, B, T, D, sources, valid, R, region_size, packed_keys,
                                                 packed_logits, static_cast<hipStream_t>(stream)));
}

int irb_summarize_region_payload(const void* packed_keys, const void* packed_logits, int dtype, const uint8_t* valid,
                                 int B, int R, int region_size, int D, uint16_t* summary, void* stream) {
  const char* fn = "irb_summarize_region_payload";
  if (int r = check_dtype(fn, dtype)) return r;
  if (B < 1 || R < 0 || region_size < 1 || D < 1) return fail(IRB_ERR_INVALID, "%s: bad sizes", fn);
  if (!packed_keys || !packed_logits || !valid || !summary) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (R == 0) return ok();
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_summarize(packed_keys, packed_logits, dtype, valid, B, R, region_size, D, summary,
                                            static_cast<hipStream_t>(stream)));
}

size_t irb_select_regions_csa_workspace_size(int B, int S, int topk, int num_docs) {
  if (B < 1 || S < 1 || topk < 1 || num_docs < 0) return 0;
  return irb::region_ids_workspace_bytes(B, S, topk, num_docs);
}

int irb_select_regions_csa(const irb_layout* layout, const float* scores, int64_t score_row_stride, int q0, int q1,
                           const int32_t* cu_blocks, int c, int topk, int32_t* region_ids, int32_t* cnt,
                           void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "irb_select_regions_csa";
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (c < 1) return fail(IRB_ERR_INVALID, "%s: c must be >= 1", fn);
  if (topk < 1 || topk > 4096) return fail(IRB_ERR_INVALID, "%s: topk must be in 1..4096 (got %d)", fn, topk);
  if (q0 < 0 || q1 <= q0 || q1 > L.S) return fail(IRB_ERR_INVALID, "%s: need 0 <= q0 < q1 <= S", fn);
  if (score_row_stride < 1) return fail(IRB_ERR_INVALID, "%s: score_row_stride must be >= 1", fn);
  if (!scores || !region_ids || !cnt || !workspace) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks", fn);
  if (ws_bytes < irb::region_ids_workspace_bytes(L.B, L.S, topk, L.num_docs))
    return fail(IRB_ERR_INVALID, "%s: workspace too small", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_region_ids(L, scores, score_row_stride, q0, q1, cu_blocks, c, topk, region_ids, cnt,
                                             workspace, static_cast<hipStream_t>(stream)));
}

int irb_expand_and_compact_routes(const irb_layout* layout, const int32_t* sel, const int32_t* cnt, int topk, int c,
                                  int window, const int32_t* cu_blocks, int L_width, int32_t* routes, int32_t* lens,
                                  void* stream) {
  const char* fn = "irb_expand_and_compact_routes";
  irb::Layout L;
  if (int r = check_layout(fn, layout, L)) return r;
  if (c < 1 || topk < 0 || window < 0) return fail(IRB_ERR_INVALID, "%s: need c >= 1, topk >= 0, window >= 0", fn);
  if (topk > 4096) return fail(IRB_ERR_INVALID, "%s: topk must be <= 4096 (got %d)", fn, topk);
  const int64_t need = static_cast<int64_t>(topk) * c + std::max(window, c - 1);
  if (L_width < need) return fail(IRB_ERR_INVALID, "%s: width %d < topk*c + max(window, c-1) = %lld", fn, L_width, (long long)need);
  if ((topk > 0 && (!sel || !cnt)) || !routes || !lens) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (L.cu_seqlens && !cu_blocks) return fail(IRB_ERR_INVALID, "%s: packed layout needs cu_blocks", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_expand(L, sel, cnt, topk, c, window, cu_blocks, L_width, routes, lens,
                                         static_cast<hipStream_t>(stream)));
}

int irb_compact_routes(const int32_t* ids_in, int64_t n_rows, int width, int64_t key_count, int32_t* ids_out,
                       int32_t* lens, int32_t* out_of_range, void* stream) {
  const char* fn = "irb_compact_routes";
  if (n_rows < 0 || n_rows > 0x7fffffff) return fail(IRB_ERR_INVALID, "%s: n_rows out of range", fn);
  if (width < 1 || width > 8192) return fail(IRB_ERR_INVALID, "%s: width must be in 1..8192 (got %d)", fn, width);
  if (key_count < 1 || key_count > 0x7fffffff) return fail(IRB_ERR_INVALID, "%s: key_count must be in 1..2^31-1", fn);
  if (!ids_in || !ids_out || !lens) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_compact(ids_in, n_rows, width, key_count, ids_out, lens, out_of_range,
                                          static_cast<hipStream_t>(stream)));
}

int irb_pack_region_bitmap(const int32_t* ids, int64_t rows, int slots, int regions, int32_t* bitmap, void* stream) {
  const char* fn = "irb_pack_region_bitmap";
  if (rows < 0 || rows > 0x7fffffffLL * 4) return fail(IRB_ERR_INVALID, "%s: rows out of range", fn);
  if (slots < 1) return fail(IRB_ERR_INVALID, "%s: slots must be >= 1", fn);
  if (regions < 1 || regions > 131072) return fail(IRB_ERR_INVALID, "%s: regions must be in 1..131072 (got %d)", fn, regions);
  if (rows == 0) return 0;
  if (!ids || !bitmap) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_bitmap(ids, rows, slots, regions, bitmap, static_cast<hipStream_t>(stream)));
}

size_t irb_build_block_lists_workspace_size(int B, int S_q, int S_k, int block_q, int block_k) {
  if (B < 1 || S_q < 1 || S_k < 1 || block_q < 1 || block_k < 1) return 0;
  const int64_t nqt = (S_q + block_q - 1) / block_q, nkt = (S_k + block_k - 1) / block_k;
  const int64_t fwd = nqt * ((nkt + 31) / 32), rev = nkt * ((nqt + 31) / 32);
  return static_cast<size_t>(B) * static_cast<size_t>(std::max(fwd, rev)) * 4;
}

int irb_build_block_lists(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int L_width,
                          int block_q, int block_k, int reverse, int32_t* counts, int32_t* indices, int width,
                          void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "irb_build_block_lists";
  if (B < 1 || S_q < 1 || S_k < 1 || L_width < 1) return fail(IRB_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (block_q < 1 || block_k < 1) return fail(IRB_ERR_INVALID, "%s: block sizes must be >= 1", fn);
  const int nqt = (S_q + block_q - 1) / block_q, nkt = (S_k + block_k - 1) / block_k;
  const int other = reverse ? nqt : nkt;
  if (width < other) return fail(IRB_ERR_INVALID, "%s: width %d < %d tiles", fn, width, other);
  if (ws_bytes < irb_build_block_lists_workspace_size(B, S_q, S_k, block_q, block_k))
    return fail(IRB_ERR_INVALID, "%s: workspace too small", fn);
  if (!routes || !lens || !counts || !indices || !workspace) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_block_lists(routes, lens, B, S_q, S_k, L_width, block_q, block_k, reverse ? 1 : 0, counts,
                                              indices, width, static_cast<uint32_t*>(workspace),
                                              static_cast<hipStream_t>(stream)));
}

size_t irb_split_full_blocks_workspace_size(int B, int S_q, int S_k, int block_q, int block_k) {
  return irb::split_cover_bytes(B, S_q, S_k, block_q, block_k);
}

int irb_split_full_blocks(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int L_width,
                          int block_q, int block_k, int reverse, const int32_t* counts, const int32_t* indices,
                          int width, int32_t* full_counts, int32_t* full_indices, int32_t* part_counts,
                          int32_t* part_indices, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "irb_split_full_blocks";
  if (B < 1 || S_q < 1 || S_k < 1 || L_width < 1) return fail(IRB_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (block_q < 1 || block_k < 1) return fail(IRB_ERR_INVALID, "%s: block sizes must be >= 1", fn);
  if (width < 1) return fail(IRB_ERR_INVALID, "%s: width must be >= 1", fn);
  if (!routes || !lens || !counts || !indices || !full_counts || !full_indices || !part_counts || !part_indices)
    return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if (full_indices == indices || part_indices == indices || full_indices == part_indices ||
      full_counts == counts || part_counts == counts || full_counts == part_counts)
    return fail(IRB_ERR_INVALID, "%s: outputs must not alias the input lists or each other", fn);
  const size_t need = irb::split_cover_bytes(B, S_q, S_k, block_q, block_k);
  uint32_t* cover = (need > 0 && workspace && ws_bytes >= need) ? static_cast<uint32_t*>(workspace) : nullptr;
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_split_full_blocks(routes, lens, B, S_q, S_k, L_width, block_q, block_k, reverse ? 1 : 0,
                                                    counts, indices, width, full_counts, full_indices, part_counts,
                                                    part_indices, cover, static_cast<hipStream_t>(stream)));
}

static int check_attn(const char* fn, const void* q, const void* k, const void* v, int dtype, const int64_t* strides,
                      const int32_t* routes, const int32_t* lens, int route_groups, int B, int S_q, int S_k,
                      int L_width, int Hq, int Hkv, int Dqk, int Dv, float scale, irb::AttnArgs& a) {
  if (int r = check_dtype(fn, dtype)) return r;
  if (B < 1 || S_q < 1 || S_k < 1 || L_width < 1) return fail(IRB_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(IRB_ERR_INVALID, "%s: Hq must be a multiple of Hkv", fn);
  if (Hq / Hkv > 64) return fail(IRB_ERR_INVALID, "%s: Hq/Hkv must be <= 64", fn);
  if (route_groups != 1 && route_groups != Hkv)
    return fail(IRB_ERR_INVALID, "%s: route_groups must be 1 or Hkv (got %d)", fn, route_groups);
  const bool dims_ok = dtype == IRB_BF16 ? ((Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128) || (Dqk == 576 && Dv == 512))
                                         : ((Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128));
  if (!dims_ok) return fail(IRB_ERR_INVALID, "%s: unsupported head dims (%d, %d)", fn, Dqk, Dv);
  // 0 selects the method's default 1/sqrt(Dqk) ([QSA] gathered_qsa_gqa_attention)
  if (scale == 0.f) scale = 1.f / std::sqrt(static_cast<float>(Dqk));
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(IRB_ERR_INVALID, "%s: softmax_scale must be finite and > 0 (0 = 1/sqrt(Dqk))", fn);
  if (!q || !k || !v || !strides || !routes || !lens) return fail(IRB_ERR_INVALID, "%s: NULL argument", fn);
  for (int i = 0; i < 9; ++i)
    if (strides[i] < 0) return fail(IRB_ERR_INVALID, "%s: negative stride", fn);
  if (strides[2] < Dqk || strides[5] < Dqk || strides[8] < Dv) return fail(IRB_ERR_INVALID, "%s: head stride below head dim", fn);
  // 16-byte vector loads of rows need 16-byte aligned rows
  const int esz = dtype == IRB_BF16 ? 2 : 4;
  for (int i = 0; i < 9; ++i)
    if ((strides[i] * esz) % 16) return fail(IRB_ERR_INVALID, "%s: strides must be multiples of 16 bytes", fn);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16)
    return fail(IRB_ERR_INVALID, "%s: q, k, v must be 16-byte aligned", fn);
  a.q = q; a.k = k; a.v = v;
  a.sq_b = strides[0]; a.sq_t = strides[1]; a.sq_h = strides[2];
  a.sk_b = strides[3]; a.sk_t = strides[4]; a.sk_h = strides[5];
  a.sv_b = strides[6]; a.sv_t = strides[7]; a.sv_h = strides[8];
  a.routes = routes; a.lens = lens;
  a.B = B; a.S_q = S_q; a.S_k = S_k; a.L = L_width; a.Hq = Hq; a.Hkv = Hkv; a.Dqk = Dqk; a.Dv = Dv;
  a.scale = scale; a.dtype = dtype; a.RG = route_groups;
  a.o32 = nullptr;
  return 0;
}

size_t irb_sparse_gqa_attention_fwd_workspace_size(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv,
                                                    int dtype, int route_groups) {
  if (B < 1 || S_q < 1 || S_k < 1 || L < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return 0;
  if (route_groups != 1 && route_groups != Hkv) return 0;
  irb::AttnArgs a{};
  a.B = B; a.S_q = S_q; a.S_k = S_k; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.Dqk = Dqk; a.Dv = Dv;
  a.dtype = dtype; a.RG = route_groups;
  return irb::attn_fwd_qbits_bytes(a);
}

int irb_sparse_gqa_attention_fwd(const void* q, const void* k, const void* v, int dtype, const int64_t* strides,
                                 const int32_t* routes, const int32_t* lens, int route_groups, int B, int S_q,
                                 int S_k, int L_width, int Hq, int Hkv, int Dqk, int Dv, float softmax_scale,
                                 void* out, float* lse, float* out_f32, void* workspace, size_t ws_bytes,
                                 void* stream) {
  const char* fn = "irb_sparse_gqa_attention_fwd";
  irb::AttnArgs a;
  if (int r = check_attn(fn, q, k, v, dtype, strides, routes, lens, route_groups, B, S_q, S_k, L_width, Hq, Hkv, Dqk, Dv,
                     softmax_scale, a))
    return r;
  if (!out || !lse) return fail(IRB_ERR_INVALID, "%s: NULL output", fn);
  if ((reinterpret_cast<uintptr_t>(out_f32) & 15) != 0)
    return fail(IRB_ERR_INVALID, "%s: out_f32 must be 16-byte aligned", fn);
  a.o32 = out_f32;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return fail(IRB_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_attn_fwd(a, out, lse, workspace, workspace ? ws_bytes : 0,
                                           static_cast<hipStream_t>(stream)));
}

size_t irb_sparse_gqa_attention_bwd_workspace_size(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv,
                                                    int dtype, int route_groups) {
  if (B < 1 || S_q < 1 || S_k < 1 || L < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return 0;
  if (dtype != IRB_F32 && dtype != IRB_BF16) return 0;
  if (route_groups != 1 && route_groups != Hkv) return 0;
  return irb::attn_bwd_workspace_bytes(B, S_q, S_k, L, Hq, Hkv, Dqk, Dv, dtype, route_groups);
}

int irb_sparse_gqa_attention_bwd_reads_out_f32(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv,
                                               int dtype, int route_groups) {
  if (route_groups != 1 && route_groups != Hkv) return 0;
  return irb::attn_bwd_reads_out32(B, S_q, S_k, L, Hq, Hkv, Dqk, Dv, dtype, route_groups) ? 1 : 0;
}

int irb_sparse_gqa_attention_bwd(const void* q, const void* k, const void* v, int dtype, const int64_t* strides,
                                 const float* out_f32, const void* dout, const float* lse, const int32_t* routes,
                                 const int32_t* lens, int route_groups, const int32_t* rev_counts,
                                 const int32_t* rev_indices,
                                 int rev_block_q, int rev_block_k, int rev_width, int B, int S_q, int S_k, int L_width,
                                 int Hq, int Hkv, int Dqk, int Dv, float softmax_scale, void* dq, void* dk, void* dv,
                                 void* workspace, size_t ws_bytes, int64_t* dropped_hits, void* stream) {
  const char* fn = "irb_sparse_gqa_attention_bwd";
  irb::AttnBwdArgs a;
  if (int r = check_attn(fn, q, k, v, dtype, strides, routes, lens, route_groups, B, S_q, S_k, L_width, Hq, Hkv, Dqk, Dv,
                     softmax_scale, a.f))
    return r;
  if (!dout || !lse || !rev_counts || !rev_indices || !dq || !dk || !dv) return fail(IRB_ERR_INVALID, "%s: NULL tensor", fn);
  if ((reinterpret_cast<uintptr_t>(out_f32) & 15) != 0)
    return fail(IRB_ERR_INVALID, "%s: out_f32 must be 16-byte aligned", fn);
  if (rev_block_k != 16) return fail(IRB_ERR_INVALID, "%s: rev_block_k must be 16 (got %d)", fn, rev_block_k);
  if (rev_block_q < 1) return fail(IRB_ERR_INVALID, "%s: rev_block_q must be >= 1", fn);
  if (rev_width < (S_q + rev_block_q - 1) / rev_block_q) return fail(IRB_ERR_INVALID, "%s: rev_width below the query tile count", fn);
  if (dk == dv && Dv > Dqk) return fail(IRB_ERR_INVALID, "%s: merged dk/dv needs Dv <= Dqk", fn);
  if (ws_bytes < irb::attn_bwd_workspace_bytes(B, S_q, S_k, L_width, Hq, Hkv, Dqk, Dv, dtype, route_groups))
    return fail(IRB_ERR_INVALID, "%s: workspace too small", fn);
  if (!workspace) return fail(IRB_ERR_INVALID, "%s: NULL workspace", fn);
  a.out32 = out_f32; a.dout = dout; a.lse = lse;
  a.rev_counts = rev_counts; a.rev_indices = rev_indices;
  a.rev_bq = rev_block_q; a.rev_bk = rev_block_k; a.rev_width = rev_width;
  a.dq = dq; a.dk = dk; a.dv = dv; a.ws = workspace; a.ws_bytes = ws_bytes; a.dropped = dropped_hits;
  IRB_REQUIRE_DEVICE();
  return launched(fn, irb::launch_attn_bwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
