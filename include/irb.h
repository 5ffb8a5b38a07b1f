/*
 * irb.h -- C ABI of libirb: learned-indexer routed sparse attention on AMD
 * Instinct MI355X (gfx950).
 *
 * Pipeline (one call per step):
 *   irb_compress_keys            raw index keys -> compressed block keys
 *   irb_prepare_index_queries    raw index queries -> normalised, rotated queries
 *   irb_indexer_score_tile       weighted-ReLU block scores for a query x block tile
 *   irb_select_topk_regions      top-k blocks per query (ascending, -1 suffix)
 *   irb_route_topk_fused         the two above without materialising scores
 *   irb_route_topk_fused_raw     the same from raw index queries (preparation fused)
 *   irb_expand_and_compact_routes blocks + tail + window -> ascending token routes
 *   irb_compact_routes           arbitrary signed ID lists -> ascending valid prefix
 *   irb_build_block_lists        forward (query->key) / reverse (key->query) tile lists
 *   irb_pack_region_bitmap       id rows -> region membership words
 *   irb_sparse_gqa_attention_fwd GQA attention over the routed keys only
 *   irb_sparse_gqa_attention_bwd its gradients; key/value side over reverse lists
 *
 * Sources (API reference pages, cited by title and documented symbol):
 *   [QSA]    nemo_automodel.components.models.qwen3_8_flash_next.qsa
 *   [CSA]    nemo_automodel.components.models.step5.sparse
 *   [FA4]    nemo_automodel.components.models.step5.fa4
 *   [LATENT] nemo_automodel.components.models.common.cudnn_sparse_attention
 *
 * Conventions shared by every call
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns.
 *     Host-side arguments (scalars, the layout struct, stride arrays) are
 *     read during the call only.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it and the call returns without waiting; the library never reads
 *     device memory from the host, so sizes come from host scalars.
 *   - All IDs and counts are int32.  Padding slots of ID lists hold -1
 *     ([QSA] QSARouteSelection.selected_token_ids).
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     non-zero status is returned with nothing enqueued and a message
 *     available from irb_last_error() (thread-local).  Status codes mirror
 *     the error classes of [LATENT] cudnn_sparse_attention:
 *       IRB_ERR_UNAVAILABLE  no usable gfx950 device / code object (RuntimeError)
 *       IRB_ERR_DTYPE        unsupported dtype (TypeError)
 *       IRB_ERR_INVALID      bad shape, size, stride, scale or layout (ValueError)
 *       IRB_ERR_HIP          a HIP launch or runtime call failed
 *     There is no fallback: an unsupported request is an error.
 *   - Contents of device inputs (IDs in range, cu_seqlens increasing) cannot
 *     be checked without a device->host read; kernels treat out-of-range IDs
 *     as padding where stated, and otherwise require the stated contract.
 */
#ifndef IRB_H_
#define IRB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum irb_status_code {
  IRB_OK = 0,
  IRB_ERR_UNAVAILABLE = 1,
  IRB_ERR_DTYPE = 2,
  IRB_ERR_INVALID = 3,
  IRB_ERR_HIP = 4
};

/* Element type of activation tensors.  bf16 is stored as raw 16-bit words. */
enum irb_dtype { IRB_F32 = 0, IRB_BF16 = 1 };

/*
 * Token layout of B rows of S physical tokens ([QSA] indexer forward,
 * _forward_packed, right_padded_sequence_lengths).  Exactly one of:
 *   cu_seqlens != NULL : packed documents, B must be 1; device int32
 *                        [num_docs+1], 0 = cu[0] < cu[1] < ... <= S.
 *                        Tokens at or past cu[num_docs] are padding.
 *   row_lens   != NULL : device int32 [B]; row b is one document of
 *                        row_lens[b] tokens (0..S) followed by padding.
 *   both NULL          : every row is one document of S tokens.
 * Compression groups, visibility and routes never cross a document
 * boundary; IDs are token indices within the row (packed: within the packed
 * row), block IDs are consecutive over a row's documents.
 */
typedef struct irb_layout {
  int32_t B;
  int32_t S;
  const int32_t* cu_seqlens;
  int32_t num_docs;
  const int32_t* row_lens;
} irb_layout;

/* 1 when a gfx950 device is present and the code objects load, else 0. */
int irb_is_available(void);
/* Message of the last failed call on this thread ("" if none). */
const char* irb_last_error(void);
const char* irb_version(void);

/*
 * a1 -- [QSA] Qwen3_8_FlashNextQSAIndexer (class docstring): every complete
 * group of c consecutive raw index keys of a document is averaged in FP32,
 * RMS-normalised (u = m * rsqrt(mean(m^2) + eps) * gamma) and rotated with
 * the rotary row of the group's FIRST token ([QSA] apply_qsa_rope: row =
 * cat(cos[D_rope/2], sin[D_rope/2]); dimension i < D_rope/2 pairs with
 * i + D_rope/2; dimensions >= D_rope pass through).  An incomplete trailing
 * group is not compressed.
 *
 *   k_idx     [B, S, D_idx] dtype, element strides (stride_b, stride_t), last dim contiguous
 *   gamma     [D_idx] fp32 gain
 *   freqs     [B, S, D_rope] fp32 contiguous, per-token document-relative rotary rows
 *   kc        OUT [B, S/c, D_idx] fp32 contiguous; block j of a row at kc[b, j];
 *             slots past the row's block count are zero
 *   cu_blocks OUT device int32 [num_docs+1] block prefix of a packed layout
 *             (cu_blocks[d] = sum_{d'<d} floor(len_d'/c)); required when
 *             packed, ignored (may be NULL) otherwise.
 * Requires 1 <= c <= 64, D_idx in {32,64,...,512} (multiple of 32),
 * D_rope even, 0 <= D_rope <= D_idx.
 */
int irb_compress_keys(const irb_layout* layout, int c, const void* k_idx, int dtype,
                      int64_t stride_b, int64_t stride_t, int D_idx, const float* gamma,
                      float eps, const float* freqs, int D_rope, float* kc, int32_t* cu_blocks,
                      void* stream);

/*
 * Index-query preparation (ahead of a2) -- [QSA] Qwen3_8_FlashNextQSAIndexer:
 * q_layernorm normalises every (token, head) row of the raw index queries
 * over the head dimension (u = x * rsqrt(mean(x^2) + eps) * gamma), and
 * apply_qsa_rope rotates it with the rotary row of the row's own token
 * (row = cat(cos[D_rope/2], sin[D_rope/2]); dimension i < D_rope/2 pairs with
 * i + D_rope/2; dimensions >= D_rope pass through).  Both steps run in FP32
 * and the result is rounded once (round-to-nearest-even) to the input dtype:
 * the normalised, rotated index queries select_qsa_token_ids expects.
 *
 *   q_raw   [n_tokens, H_idx, D_idx] dtype, contiguous, 16-byte aligned
 *   gamma   [D_idx] fp32 gain
 *   rope    [n_tokens, D_rope] fp32 contiguous rotary rows, built at each token's
 *           document-relative position (may be NULL when D_rope == 0)
 *   q_out   OUT [n_tokens, H_idx, D_idx] dtype, 16-byte aligned; may alias q_raw
 * Requires D_idx in {32, 64, 128, 256, 512}, D_rope even, 0 <= D_rope <= D_idx,
 * eps >= 0.  A batch [B, S, ...] is n_tokens = B * S.  n_tokens == 0 is a no-op.
 */
int irb_prepare_index_queries(const void* q_raw, int dtype, int64_t n_tokens, int H_idx, int D_idx,
                              const float* gamma, float eps, const float* rope, int D_rope, void* q_out,
                              void* stream);

/*
 * a2 -- [CSA] indexer_score_tile (weighted-ReLU scoring into one bounded FP32
 * tile, signed FP32 head weights) with the visibility rule of [QSA]
 * select_qsa_token_ids (query at document position p sees the first
 * floor((p+1)/c) complete blocks of its own document):
 *     out[b, t-q0, j-j0] = score_scale * sum_h w[b,t,h] * max(0, q[b,t,h,:] . kc[b,j,:])
 * for visible j, and -inf otherwise (padding queries: all -inf).
 * The products use bf16 MFMA with kc split into bf16 high+low parts and FP32
 * accumulation (fp32 queries are split the same way).  score_scale = 0
 * selects the default 1/sqrt(D_idx) ([QSA] select_qsa_token_ids); otherwise
 * it must be finite and > 0.
 *
 *   q_idx  [B, S, H_idx, D_idx] dtype contiguous
 *   w      [B, S, H_idx] fp32 contiguous
 *   kc     [B, S/c, D_idx] fp32 (as written by irb_compress_keys)
 *   cu_blocks as written by irb_compress_keys (packed layouts), else NULL
 *   out    OUT fp32, element (b, t-q0, j-j0) at out[(b*(q1-q0) + t-q0)*out_row_stride + j-j0]
 * Requires 0 <= q0 < q1 <= S, 0 <= j0 < j1 <= S/c, out_row_stride >= j1-j0,
 * H_idx in {4, 8, 16, 32, 48, 64}, D_idx in {32, 64, 128}.
 */
int irb_indexer_score_tile(const irb_layout* layout, const void* q_idx, int dtype, int H_idx,
                           int D_idx, const float* w, const float* kc, const int32_t* cu_blocks,
                           int c, float score_scale, int q0, int q1, int j0, int j1, float* out,
                           int64_t out_row_stride, void* stream);

/*
 * a3 -- [QSA] select_qsa_token_ids (the best budget/c blocks) and [CSA]
 * RegionMetadata.dense_region_ids / RegionSelection.region_ids: each valid
 * query t in [q0, q1) takes k_eff = min(topk, nb(t)) of its visible blocks
 * with the largest scores; equal scores go to the lower block ID, -0.0 and
 * +0.0 are equal, NaN ranks below -inf.  IDs are written ascending, then -1.
 * Padding queries: cnt = 0, all -1.
 *
 *   scores  fp32 rows for queries q0..q1-1; row r at scores + (b*(q1-q0)+r)*score_row_stride,
 *           column j = block ID j (the tile must start at block 0 and cover
 *           every block visible to its rows)
 *   sel     OUT [B, S, topk] int32 (rows q0..q1-1 written)
 *   cnt     OUT [B, S] int32 (rows q0..q1-1 written)
 * Requires 1 <= topk <= 4096, 1 <= c.
 */
int irb_select_topk_regions(const irb_layout* layout, const float* scores, int64_t score_row_stride,
                            int q0, int q1, const int32_t* cu_blocks, int c, int topk, int32_t* sel,
                            int32_t* cnt, void* stream);

/*
 * a2+a3 in one call: the same sel/cnt as irb_indexer_score_tile followed by
 * irb_select_topk_regions over [q0, q1), with the FP32 scores of at most a
 * bounded number of query rows alive at a time ([QSA] select_qsa_token_ids:
 * chunking bounds the score temporary without changing top-k semantics).
 * workspace: device scratch; irb_route_topk_fused_workspace_size() gives the
 * compressed keys split into bf16 high/low rows (B * (S/c) * D_idx * 4 bytes,
 * rounded up to 256) plus a 256 MiB-budget of score rows; any size holding
 * the split keys and at least one score row works (rows per chunk = the rest
 * / (B * (S/c) * 4)).
 */
size_t irb_route_topk_fused_workspace_size(int B, int S, int c, int D_idx, int topk, int q0, int q1);
int irb_route_topk_fused(const irb_layout* layout, const void* q_idx, int dtype, int H_idx,
                         int D_idx, const float* w, const float* kc, const int32_t* cu_blocks,
                         int c, float score_scale, int topk, int q0, int q1, int32_t* sel,
                         int32_t* cnt, void* workspace, size_t ws_bytes, void* stream);

/*
 * Index-query preparation fused into a2+a3 -- [QSA] Qwen3_8_FlashNextQSAIndexer
 * (q_layernorm, apply_qsa_rope) feeding select_qsa_token_ids: the same
 * sel/cnt as irb_prepare_index_queries(q_raw -> q) followed by
 * irb_route_topk_fused(q), without writing or re-reading the prepared
 * queries.  The score kernel normalises and rotates each raw query row as it
 * loads it, with the preparation call's FP32 arithmetic in the same order
 * and the same single rounding to the input dtype, so its operands equal the
 * prepared queries bit for bit.
 *   q_raw  [B, S, H_idx, D_idx] dtype contiguous, 16-byte aligned (raw index queries)
 *   gamma  [D_idx] fp32 gain, 16-byte aligned;  eps >= 0
 *   rope   [B, S, D_rope] fp32 rotary rows cat(cos, sin) at each token's
 *          document position, 16-byte aligned (NULL when D_rope == 0)
 *   everything else, the workspace included, as irb_route_topk_fused
 *          (irb_route_topk_fused_workspace_size gives its size).
 * Requires D_rope = 0 or a multiple of 64 up to D_idx (each lane of the score
 * kernel then holds the rotation partners of its own dimensions); other
 * rotary widths go through irb_prepare_index_queries + irb_route_topk_fused.
 */
int irb_route_topk_fused_raw(const irb_layout* layout, const void* q_raw, int dtype, int H_idx, int D_idx,
                             const float* gamma, float eps, const float* rope, int D_rope, const float* w,
                             const float* kc, const int32_t* cu_blocks, int c, float score_scale, int topk, int q0,
                             int q1, int32_t* sel, int32_t* cnt, void* workspace, size_t ws_bytes, void* stream);

/*
 * irb_route_topk_fused without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and results as
 * irb_route_topk_fused, minus the workspace: the split keys and score rows
 * live in a static device array of IRB_NOALLOC_SCRATCH_BYTES that each GPU
 * the library runs on holds until the process ends.  The call allocates
 * nothing; it needs B * (S/c) * D_idx * 4 bytes (rounded up to 256) of split
 * keys plus at least one B * (S/c) * 4-byte score row within that maximum,
 * and returns IRB_ERR_INVALID otherwise (e.g. B * (S/c) = 16384 blocks of
 * 128 dims use 8 MiB, leaving 56 MiB of score rows; score chunks hold as many
 * query rows as fit).  The scratch needs no clearing between calls.  All
 * calls on one GPU share that GPU's array: calls that overlap in time on one
 * GPU (different streams or host threads without ordering) race and give
 * wrong selections; calls ordered on one stream are safe.
 */
#define IRB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int irb_route_topk_fused_noalloc(const irb_layout* layout, const void* q_idx, int dtype, int H_idx,
                                 int D_idx, const float* w, const float* kc, const int32_t* cu_blocks,
                                 int c, float score_scale, int topk, int q0, int q1, int32_t* sel,
                                 int32_t* cnt, void* stream);

/*
 * a2 / a2+a3 with one score row and one selection per KV group -- [CSA]
 * indexer_score_tile: index queries [batch, queries, groups, heads, dim] and
 * signed weights [batch, queries, groups, heads] score the shared region
 * summaries into FP32 tiles [batch, groups, queries, regions]; selections
 * and bitmaps carry the same groups axis (pack_region_bitmap).  Group g's
 * score is the ungrouped score over its own H_idx heads:
 *     out[g, b, t-q0, j-j0] = score_scale * sum_h w[b,t,g,h] * max(0, q[b,t,g,h,:] . kc[b,j,:])
 *
 *   q_idx  [B, S, groups, H_idx, D_idx] dtype contiguous
 *   w      [B, S, groups, H_idx] fp32 contiguous
 *   out    OUT group g's tile at out + g * B * (q1-q0) * out_row_stride, laid
 *          out as irb_indexer_score_tile's
 *   sel    OUT [groups, B, S, topk] int32, cnt OUT [groups, B, S] int32
 *          (group-major: each group's selection is one [B, S, topk] block,
 *          which irb_expand_and_compact_routes expands into that group's
 *          [B, S, L] routes; for B = 1 the CSA page's [batch, groups, ...])
 *   workspace: irb_route_topk_fused_groups_workspace_size() bytes (the split
 *          keys once, score rows of every group); any size holding the split
 *          keys and one score row per group works.
 * bf16 queries with 4 or 8 heads per group, groups * heads in {16, 32} and
 * D_idx in {64, 128} score every group in one launch (a lane's four
 * accumulator rows are one group's heads, or half of them); other shapes
 * score the groups one after another with the ungrouped kernels.
 * Requires 1 <= groups <= 64; everything else as for the ungrouped calls.
 */
size_t irb_route_topk_fused_groups_workspace_size(int B, int S, int c, int D_idx, int topk, int q0, int q1,
                                                  int groups);
int irb_indexer_score_tile_groups(const irb_layout* layout, const void* q_idx, int dtype, int groups,
                                  int H_idx, int D_idx, const float* w, const float* kc,
                                  const int32_t* cu_blocks, int c, float score_scale, int q0, int q1,
                                  int j0, int j1, float* out, int64_t out_row_stride, void* stream);
int irb_route_topk_fused_groups(const irb_layout* layout, const void* q_idx, int dtype, int groups,
                                int H_idx, int D_idx, const float* w, const float* kc,
                                const int32_t* cu_blocks, int c, float score_scale, int topk, int q0,
                                int q1, int32_t* sel, int32_t* cnt, void* workspace, size_t ws_bytes,
                                void* stream);

/*
 * Step-5 CSA variant (next row of the hot path) -- [CSA] nemo_automodel.
 * components.models.step5.sparse.  Regions are summarised by learned
 * per-dimension weights instead of mean pooling, scoring takes E4M3-rounded
 * BF16 queries and summaries (irb_indexer_score_tile accepts them as bf16
 * tensors and reproduces their products exactly), and the selection keeps
 * the query's current region in an extra slot.
 *
 * irb_round_e4m3 -- the E4M3 rounding of [CSA] indexer_score_tile's inputs:
 *   out[i] = x[i] rounded to nearest even on the E4M3 grid (4 exponent bits,
 *   bias 7, 3 mantissa bits, largest 448; a value rounding past it, or not
 *   finite, gives NaN), stored as bf16 (exact).  x bf16 or fp32 [n];
 *   out bf16 [n] (may alias a bf16 x).
 */
int irb_round_e4m3(const void* x, int dtype, int64_t n, uint16_t* out, void* stream);

/*
 * [CSA] gather_region_payload / _gather_region_payload: the keys and
 * compression logits of every region's source tokens, gathered without
 * arithmetic (bit-exact copies):
 *   packed_keys[b, r, s, :] = keys[b, sources[b, r, s], :] where the slot is
 *   valid, zeros otherwise; packed_logits likewise.
 *   keys, logits [B, T, D] dtype contiguous; sources int32 [B, R, region_size]
 *   (-1 = missing slot; ids outside [0, T) count as missing); valid uint8
 *   [B, R, region_size] (0 excludes a padding token; NULL = every slot with
 *   a source); outputs [B, R, region_size, D] dtype.  Requires D * element
 *   size a multiple of 16 and 16-byte aligned keys, logits and outputs.
 */
int irb_gather_region_payload(const void* keys, const void* logits, int dtype, int B, int T, int D,
                              const int32_t* sources, const uint8_t* valid, int R, int region_size,
                              void* packed_keys, void* packed_logits, void* stream);

/*
 * [CSA] _summarize_region_payload: FP32 arithmetic and the two quantisation
 * roundings the page requires.  The page does not print the formula; the
 * reading taken here: per region r and dimension d,
 *   s[b, r, d] = sum_s softmax_s(z[b, r, s, d]) k[b, r, s, d]
 * over the region's valid slots (the softmax of the per-dimension
 * compression logits, max-subtracted), in FP32, rounded to BF16 and then to
 * E4M3 (irb_round_e4m3).  A region with no valid slot gives 0.
 *   packed_keys, packed_logits [B, R, region_size, D] dtype contiguous (as
 *   irb_gather_region_payload writes them); valid uint8 [B, R, region_size];
 *   summary OUT bf16 [B, R, D] holding E4M3 values.
 */
int irb_summarize_region_payload(const void* packed_keys, const void* packed_logits, int dtype,
                                 const uint8_t* valid, int B, int R, int region_size, int D,
                                 uint16_t* summary, void* stream);

/*
 * [CSA] RegionSelection.region_ids with RegionMetadata.current: for each
 * valid query t in [q0, q1) at document position pos, its historical
 * regions -- the floor(pos / c) complete blocks of its document before the
 * one holding it -- compete for topk slots by score exactly as in
 * irb_select_topk_regions; the current region (floor(pos / c) of its
 * document) is always added.  The ids are the page's region numbering, in
 * which every token belongs to a region, so each document's regions (its
 * incomplete last one included) are consecutive: written ascending (the
 * current one last), then the sentinel R = the row's region count up to
 * topk + 1 slots; cnt = used slots (0 for padding queries, which hold only
 * sentinels).
 *   scores   as for irb_select_topk_regions (block columns of this library's
 *            numbering: complete blocks only, e.g. irb_indexer_score_tile)
 *   region_ids OUT [B, S, topk + 1] int32; cnt OUT [B, S] int32 (rows q0..q1-1)
 *   workspace irb_select_regions_csa_workspace_size() bytes of device scratch
 * Requires 1 <= topk <= 4096, 1 <= c.
 */
size_t irb_select_regions_csa_workspace_size(int B, int S, int topk, int num_docs);
int irb_select_regions_csa(const irb_layout* layout, const float* scores, int64_t score_row_stride,
                           int q0, int q1, const int32_t* cu_blocks, int c, int topk, int32_t* region_ids,
                           int32_t* cnt, void* workspace, size_t ws_bytes, void* stream);

/*
 * a4 -- [QSA] select_qsa_token_ids: selected blocks expand to their c token
 * IDs, then the tokens of the current incomplete group [doc_start + nb*c, t]
 * are appended; plus the window [max(doc_start, t-window+1), t] ([CSA]
 * RegionMetadata.window_layout: the query and at most window-1 earlier keys).
 * The union is written ascending without duplicates ([QSA] qsa_gqa_attention:
 * duplicates collapse), then -1 up to width L; lens[t] = its size.
 *
 *   sel, cnt  [B, S, topk] / [B, S] as written by irb_select_topk_regions
 *   routes    OUT [B, S, L] int32;  lens OUT [B, S] int32
 * Requires L >= topk*c + max(window, c-1) (the [QSA] width budget + c - 1 when
 * window == 0), window >= 0, 0 <= topk <= 4096 (sel and cnt may be NULL when
 * topk == 0).
 */
int irb_expand_and_compact_routes(const irb_layout* layout, const int32_t* sel, const int32_t* cnt,
                                  int topk, int c, int window, const int32_t* cu_blocks, int L,
                                  int32_t* routes, int32_t* lens, void* stream);

/*
 * a4 (compaction) -- [LATENT] _compact_and_sort_indices: each row of `width`
 * signed IDs becomes its ascending, duplicate-free valid prefix (valid =
 * 0 <= id < key_count) followed by -1; lens[r] = prefix length.  IDs at or
 * past key_count are dropped and counted into *out_of_range (device int32,
 * nullable; incremented, so zero it first).
 *
 *   ids_in [n_rows, width] int32, ids_out OUT [n_rows, width], lens OUT [n_rows]
 * Requires 1 <= width <= 8192, 1 <= key_count < 2^31.  ids_in == ids_out is allowed.
 */
int irb_compact_routes(const int32_t* ids_in, int64_t n_rows, int width, int64_t key_count,
                       int32_t* ids_out, int32_t* lens, int32_t* out_of_range, void* stream);

/*
 * Route bitmap -- [CSA] pack_region_bitmap: each row of int32 region ids
 * becomes ceil(regions / 32) membership words, bit r % 32 of word r / 32 set
 * exactly when region r occurs in the row, packed without any scatter
 * workspace.  Ids at or above `regions` are padding, as on the page; negative
 * ids are padding too (this library pads route lists with -1).  Repeats are
 * allowed and the rows need not be sorted.  Words hold the bit pattern as int32.
 *
 *   ids     [rows, slots] int32 (any leading shape flattened to rows)
 *   bitmap  OUT [rows, ceil(regions / 32)] int32; every word is written
 * Requires slots >= 1, 1 <= regions <= 131072.  rows == 0 is a no-op.
 */
int irb_pack_region_bitmap(const int32_t* ids, int64_t rows, int slots, int regions, int32_t* bitmap,
                           void* stream);

/*
 * a5 -- [FA4] _block_lists / _selected_block_lists / _BackwardBlockPartition:
 * block lists from token routes without a dense grid in HBM.
 *   reverse == 0: rows = ceil(S_q/block_q) query tiles; row i lists, ascending,
 *                 the key tiles floor(k/block_k) holding a routed key of one
 *                 of its queries.
 *   reverse == 1: rows = ceil(S_k/block_k) key tiles; row j lists, ascending,
 *                 the query tiles that route to it (key-to-query lists used
 *                 by the backward pass).
 *   routes [B, S_q, L], lens [B, S_q] (ascending valid prefixes)
 *   counts OUT [B, rows] int32; indices OUT [B, rows, width] int32, -1 after the count
 *   workspace: irb_build_block_lists_workspace_size() bytes of device scratch
 * Requires width >= number of tiles on the other axis, block_q, block_k >= 1.
 */
size_t irb_build_block_lists_workspace_size(int B, int S_q, int S_k, int block_q, int block_k);
int irb_build_block_lists(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int L,
                          int block_q, int block_k, int reverse, int32_t* counts, int32_t* indices,
                          int width, void* workspace, size_t ws_bytes, void* stream);

/*
 * Full/partial block split -- [FA4] _split_forward_full_blocks and
 * _split_backward_full_blocks (_BackwardBlockPartition: independent partial
 * and full counts and index lists in the input layouts): the entries of a
 * forward or reverse block list from irb_build_block_lists (same routes,
 * block sizes and direction) are separated, each list's order kept, into
 * full blocks -- every (query, key) pair of the block's rectangle
 * [i*block_q, min((i+1)*block_q, S_q)) x [j*block_k, min((j+1)*block_k, S_k))
 * is routed, so the block needs no mask -- and partial ones.  The page proves
 * fullness for the complete causal rectangles of an all-selected query
 * prefix; this call tests the routes themselves, which covers that case and
 * any other fully routed block (a window, a dense selection).
 *
 *   routes [B, S_q, L], lens [B, S_q] (ascending unique valid prefixes)
 *   counts [B, rows], indices [B, rows, width] as irb_build_block_lists wrote them
 *   full_counts, part_counts OUT [B, rows]; full_indices, part_indices OUT
 *     [B, rows, width] int32; entries past each count are not written (as
 *     for the page's lists, readers ignore them).  Outputs must not alias
 *     the inputs or each other.
 *   workspace: optional device scratch.  With block_q = 1 and at least
 *     irb_split_full_blocks_workspace_size() bytes (one bit per (query, key
 *     tile)), every route is read once and marks the key tiles it holds
 *     completely, and each listed block tests one bit; otherwise (NULL, too
 *     small, or block_q > 1) every (block, query) pair binary-searches the
 *     query's route.  Results are the same.
 * Per-KV-group routes [RG, B, S_q, L] are RG * B route rows.
 * Requires block_q, block_k, width >= 1.
 */
size_t irb_split_full_blocks_workspace_size(int B, int S_q, int S_k, int block_q, int block_k);
int irb_split_full_blocks(const int32_t* routes, const int32_t* lens, int B, int S_q, int S_k, int L,
                          int block_q, int block_k, int reverse, const int32_t* counts,
                          const int32_t* indices, int width, int32_t* full_counts, int32_t* full_indices,
                          int32_t* part_counts, int32_t* part_indices, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * a6 -- [QSA] gathered_qsa_gqa_attention / qsa_gqa_attention and [LATENT]
 * cudnn_sparse_attention: every valid query attends only to the keys at
 * routes[b, t, 0:lens[b,t]]; query head h uses KV head h / (Hq/Hkv)
 * (consecutive heads share a group):
 *     o = softmax(softmax_scale * q K_R^T) V_R,  lse = logsumexp(scale * q K_R^T)
 * A query with lens = 0 gets o = 0 and lse = -inf.  Softmax and both
 * products accumulate in FP32; o is rounded once to the input dtype.
 * softmax_scale = 0 selects the default 1/sqrt(Dqk); otherwise it must be
 * finite and > 0.
 *
 *   q [B, S_q, Hq, Dqk], k [B, S_k, Hkv, Dqk], v [B, S_k, Hkv, Dv]: dtype,
 *     element strides strides[0..2] = q (batch, token, head), [3..5] = k,
 *     [6..8] = v; the last dimension is contiguous.  A latent layout passes
 *     v = k (the value is the first Dv channels of each key row).
 *   routes [RG, B, S_q, L] int32, lens [RG, B, S_q] int32 with RG =
 *     route_groups: routes[g,b,t,0:lens] ascending, unique, in [0, S_k).
 *     RG = 1: one route per query, read by every head.  RG = Hkv: one route
 *     per KV group and query ([CSA] indexer_score_tile / pack_region_bitmap:
 *     scores and selections carry a groups axis; [FA4] _provider_heads: a
 *     group's metadata serves the consecutive query heads sharing its KV
 *     head), read by the heads h with h / (Hq/Hkv) = g.  Group-major, so each
 *     group's routes are one [B, S_q, L] block (for B = 1 the CSA page's
 *     [batch, groups, queries, slots]).
 *   out OUT [B, S_q, Hq, Dv] dtype contiguous; lse OUT [B, Hq, S_q] fp32
 *   out_f32 OUT, nullable: [B, S_q, Hq, Dv] fp32 contiguous, 16-byte aligned:
 *     o before its rounding to the input dtype -- what the backward's
 *     row statistic Delta = rowsum(dO * o) is read off (irb_sparse_gqa_
 *     attention_bwd's out_f32), saving it a pass over the routes
 *   workspace: optional device scratch (16-byte aligned, NULL allowed) of
 *     irb_sparse_gqa_attention_fwd_workspace_size() bytes: the key-membership
 *     words of every route row ([FA4] _block_lists builds its block masks
 *     from the routes once; here one bit per (route row, key)), built once
 *     per call and read by every KV head's query tiles.  The size is 0 where
 *     the query-tile kernel does not run (fp32, head dims 576/512, group
 *     sizes other than 4, 8, 16) or the words would exceed 256 MiB; with no
 *     (or a smaller) workspace the tiles build their masks from the routes
 *     in LDS.  Results are the same either way.
 * Requires Hq % Hkv == 0, Hq/Hkv <= 64, (Dqk, Dv) in {(64,64), (128,128)} or,
 * for bf16, (576,512); strides and q/k/v addresses 16-byte aligned;
 * route_groups = 1 or Hkv.
 */
size_t irb_sparse_gqa_attention_fwd_workspace_size(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk,
                                                   int Dv, int dtype, int route_groups);
int irb_sparse_gqa_attention_fwd(const void* q, const void* k, const void* v, int dtype,
                                 const int64_t* strides, const int32_t* routes, const int32_t* lens,
                                 int route_groups, int B, int S_q, int S_k, int L, int Hq, int Hkv,
                                 int Dqk, int Dv, float softmax_scale, void* out, float* lse, float* out_f32,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * a7 -- gradients of irb_sparse_gqa_attention_fwd ([QSA]
 * gathered_qsa_gqa_attention is the differentiable reference; the indexer is
 * frozen, so only q, k and v receive gradients):
 *     P = exp(scale q K_R^T - lse), dP = dO V_R^T, Delta = rowsum(dO * o),
 *     dS = P (dP - Delta), dq = scale dS K_R, dK += scale dS^T q, dV += P^T dO.
 * dq is computed per query over its route; dK and dV per key tile over the
 * reverse lists ([FA4] _selected_block_lists, reverse): rev_counts /
 * rev_indices from irb_build_block_lists(reverse=1) with the same
 * rev_block_q, rev_block_k.  No atomics: results are deterministic.
 * With route_groups = Hkv the reverse lists are those of the grouped routes
 * viewed as RG * B rows (irb_build_block_lists with B' = RG * B): counts
 * [RG, B, key tiles], indices [RG, B, key tiles, rev_width]; KV head g reads
 * group g's lists and routes.
 *
 *   out_f32    nullable: the forward's FP32 output (irb_sparse_gqa_attention_fwd
 *              out_f32).  Given, Delta = rowsum(dO * o) is read off it for the
 *              sizes where irb_sparse_gqa_attention_bwd_reads_out_f32 is 1;
 *              otherwise (or NULL) Delta is formed with o in FP32 from the
 *              routes (the query side sums P dP, or the forward runs again in
 *              Delta mode) -- never from the stored, rounded output, whose
 *              rounding would enter every dS.  16-byte aligned.
 *   lse        the forward's lse; dout [B, S_q, Hq, Dv] dtype contiguous
 *   dq OUT [B, S_q, Hq, Dqk] dtype contiguous
 *   dk OUT [B, S_k, Hkv, Dqk] dtype contiguous, dv OUT [B, S_k, Hkv, Dv]
 *     dtype contiguous.  dk == dv (latent: v aliases k) writes the merged
 *     gradient dK + [dV, 0] into dk.
 *   workspace: irb_sparse_gqa_attention_bwd_workspace_size() bytes of device
 *     scratch (same B, S_q, S_k, L, heads, dims, dtype and route_groups as
 *     the call).  For bf16 with Dqk = Dv in {64, 128} it holds, per route
 *     group and 16-key tile, the listed queries whose routes reach the tile
 *     with their 16-bit key masks (at most RG * B * S_q * min(L, ceil(S_k /
 *     16)) entries; lists that repeat a query tile, or stale lists, can
 *     overflow it: entries past it are dropped and counted), and per group
 *     of four such tiles the union of their lists (bounded by the routes)
 *     and the order in which the key-side workgroups are dispatched.
 *   dropped_hits OUT device int64 scalar, nullable: written with the number
 *     of hit entries that did not fit the workspace (0 for consistent
 *     routes and reverse lists; a non-zero value means dk / dv miss those
 *     contributions).  Always written when given.
 * Requirements as for the forward, plus rev_block_k = 16.
 */
size_t irb_sparse_gqa_attention_bwd_workspace_size(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk,
                                                   int Dv, int dtype, int route_groups);
/*
 * 1 when irb_sparse_gqa_attention_bwd with these sizes reads Delta off an
 * out_f32 given to it -- a pass over the routes (or a forward in Delta mode)
 * is then saved, so a training step should have the forward write out_f32 --
 * and 0 where its per-query dQ pass forms Delta anyway (the FP32 output would
 * only cost its write).  Contiguous q / k / v assumed; 0 for invalid sizes.
 */
int irb_sparse_gqa_attention_bwd_reads_out_f32(int B, int S_q, int S_k, int L, int Hq, int Hkv, int Dqk, int Dv,
                                               int dtype, int route_groups);
int irb_sparse_gqa_attention_bwd(const void* q, const void* k, const void* v, int dtype,
                                 const int64_t* strides, const float* out_f32, const void* dout,
                                 const float* lse, const int32_t* routes, const int32_t* lens,
                                 int route_groups, const int32_t* rev_counts, const int32_t* rev_indices,
                                 int rev_block_q, int rev_block_k, int rev_width, int B, int S_q,
                                 int S_k, int L, int Hq, int Hkv, int Dqk, int Dv,
                                 float softmax_scale, void* dq, void* dk, void* dv, void* workspace,
                                 size_t ws_bytes, int64_t* dropped_hits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IRB_H_ */
