"""Plain FP64 CPU oracle for learned-indexer routed sparse attention.

TEST INFRASTRUCTURE.  Nothing on the product path may import, call or execute
this package: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP library or its Python
binding and imports neither.

Every function evaluates the plain definition of one step of the method in
float64 NumPy, with no blocking, fusion or reordering beyond what the
definition states.  Sources, cited by page title and documented symbol:

* QSA page   -- nemo_automodel.components.models.qwen3_8_flash_next.qsa
* CSA page   -- nemo_automodel.components.models.step5.sparse
* FA4 page   -- nemo_automodel.components.models.step5.fa4
* layers page-- nemo_automodel.components.models.step5.layers
* latent page-- nemo_automodel.components.models.common.cudnn_sparse_attention

Readings taken where the pages are silent or disagree (each is listed with
its reason in the design notes):

* scores are ``scale * sum_h w[t,h] * relu(q[t,h] . k[j])`` -- the QSA page's
  unweighted sum with the CSA page's signed FP32 head weights; ``w == 1``
  and ``scale = 1/sqrt(D_idx)`` give the QSA formula exactly;
* ties in top-k go to the lower block ID; -0.0 equals +0.0;
* a window of ``W`` tokens ends at and includes the query itself;
* RMSNorm gain is multiplicative; RoPE pairs dimension ``i`` with
  ``i + D_rope/2`` (half split), dimensions >= D_rope pass through;
* padding queries get all -1 routes and zero attention output, lse = -inf;
  a query with an empty route likewise;
* latent attention uses the first ``Dv`` channels of the shared latent row
  as the value, and its key/value gradients land in the same buffer;
* per-KV-group routes are laid out group-major, [R, B, S, L] with R = 1
  (one route shared by every head) or R = Hkv (one per KV group); for B = 1
  this is the CSA page's [batch, groups, queries, slots].

* CSA variant: slots of a region that are not valid hold zeros in the
  gathered payload; a region summary is the per-dimension softmax (over the
  region's valid slots) of the compression logits weighting the keys, in
  float32, rounded to BF16 and then to E4M3 (E4M3 as torch's float8_e4m3fn
  conversion: round to nearest even, NaN past 448); a query's historical
  regions are the complete ones before the region holding it, and that
  current region fills the extra selection slot.

Parity status: every function here is pinned by the CPU tests (hand-derived
fixtures, brute force, library special cases, invariants) with respect to
these readings.  ``summarize_region_payload`` is "parity unpinned" with
respect to the pages: the CSA page states its precision (FP32 arithmetic,
BF16 then E4M3 rounding) but not its formula, so only the reading above is
pinned (closed forms: equal logits give the mean, a lone or dominant slot
gives its key, the BF16 rounding precedes the E4M3 one).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------

def documents(B: int, S: int, cu_seqlens: Optional[np.ndarray] = None,
              row_lens: Optional[np.ndarray] = None):
    """Documents of every batch row as lists of (start, stop).

    Packed layout (QSA page, ``_forward_packed``): one row, documents given
    by strictly increasing ``cu_seqlens`` starting at 0; tokens at or beyond
    the last boundary are padding.  Right-padded layout (QSA page,
    ``right_padded_sequence_lengths``): row ``b`` is one document of length
    ``row_lens[b]`` followed by padding.  Neither: each row one document.
    """
    if cu_seqlens is not None:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        if B != 1:
            raise ValueError("packed layout needs B == 1")
        if cu[0] != 0 or any(b <= a for a, b in zip(cu, cu[1:])) or cu[-1] > S:
            raise ValueError("cu_seqlens must start at 0, increase strictly and end <= S")
        return [[(cu[d], cu[d + 1]) for d in range(len(cu) - 1)]]
    rows = []
    for b in range(B):
        n = S if row_lens is None else int(row_lens[b])
        if not 0 <= n <= S:
            raise ValueError("row length out of range")
        rows.append([(0, n)] if n > 0 else [])
    return rows


def block_bases(docs, c: int):
    """Global block ID of the first complete block of every document.

    Packed rows number blocks consecutively over documents (the CSA page's
    global region IDs); each document contributes ``floor(len / c)`` blocks
    (QSA page, indexer class: only complete groups are compressed).
    """
    out = []
    for row in docs:
        base, bases = 0, []
        for (a, e) in row:
            bases.append(base)
            base += (e - a) // c
        out.append(bases)
    return out


def token_info(docs, S: int, c: int):
    """Per token: (valid, doc_start, block_base, nb) with nb = floor((pos+1)/c).

    ``nb`` is the number of complete blocks visible to the query at
    document-relative position ``pos`` (QSA page, ``select_qsa_token_ids``).
    """
    B = len(docs)
    valid = np.zeros((B, S), dtype=bool)
    start = np.zeros((B, S), dtype=np.int64)
    base = np.zeros((B, S), dtype=np.int64)
    nb = np.zeros((B, S), dtype=np.int64)
    bases = block_bases(docs, c)
    for b, row in enumerate(docs):
        for d, (a, e) in enumerate(row):
            valid[b, a:e] = True
            start[b, a:e] = a
            base[b, a:e] = bases[b][d]
            nb[b, a:e] = (np.arange(e - a) + 1) // c
    return valid, start, base, nb


# ---------------------------------------------------------------------------
# a1: key compression
# ---------------------------------------------------------------------------

def compress_keys(kI, gamma, eps, freqs, c, cu_seqlens=None, row_lens=None, d_rope=None):
    """Compressed index keys [B, S//c, D] (float64) and block bases.

    QSA page, indexer class: complete consecutive groups of ``c`` raw index
    keys are averaged, then RMS-normalised (gain ``gamma``, variance epsilon
    ``eps``) and rotated at the group's first token.  ``apply_qsa_rope``:
    the table row is ``cat(cos, sin)`` of width ``D_rope``; dimensions from
    ``D_rope`` on pass through.  ``_forward_packed``: groups restart at each
    document start.  Unused block slots are zero.
    """
    kI = np.asarray(kI, dtype=np.float64)
    B, S, D = kI.shape
    freqs = np.asarray(freqs, dtype=np.float64)
    R = freqs.shape[-1] if d_rope is None else d_rope
    half = R // 2
    g = np.asarray(gamma, dtype=np.float64)
    docs = documents(B, S, cu_seqlens, row_lens)
    bases = block_bases(docs, c)
    kc = np.zeros((B, S // c, D), dtype=np.float64)
    for b, row in enumerate(docs):
        for d, (a, e) in enumerate(row):
            n = (e - a) // c
            if n == 0:
                continue
            groups = kI[b, a:a + n * c].reshape(n, c, D)
            m = groups.mean(axis=1)
            u = m / np.sqrt(np.mean(m * m, axis=1, keepdims=True) + eps) * g
            first = a + c * np.arange(n)
            cos = freqs[b, first, :half]
            sin = freqs[b, first, half:2 * half]
            x1 = u[:, :half].copy()
            x2 = u[:, half:2 * half].copy()
            u[:, :half] = x1 * cos - x2 * sin
            u[:, half:2 * half] = x2 * cos + x1 * sin
            kc[b, bases[b][d]:bases[b][d] + n] = u
    cu_blocks = None
    if cu_seqlens is not None:
        total = sum((e - a) // c for (a, e) in docs[0])
        cu_blocks = np.array(bases[0] + [total], dtype=np.int32)
    return kc, cu_blocks


def prepare_index_queries(q_raw, gamma, freqs, eps=1e-5, d_rope=None):
    """Normalised, rotated index queries [..., S, H, D] (float64, not rounded).

    QSA page: the indexer's ``q_layernorm`` (RMSNorm over the head dimension,
    gain ``gamma``, variance epsilon ``eps``) normalises every (token, head)
    row of the raw index queries, and ``apply_qsa_rope`` rotates it with the
    rotary row of the query's own token (``cat(cos, sin)`` of width
    ``D_rope``; dimension ``i < D_rope/2`` pairs with ``i + D_rope/2``;
    dimensions from ``D_rope`` on pass through).  ``q_raw`` is [B, S, H, D],
    ``freqs`` [B, S, D_rope].
    """
    q = np.asarray(q_raw, dtype=np.float64)
    freqs = np.asarray(freqs, dtype=np.float64)
    R = freqs.shape[-1] if d_rope is None else d_rope
    half = R // 2
    g = np.asarray(gamma, dtype=np.float64)
    u = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps) * g
    out = u.copy()
    if half:
        cos = freqs[..., :half][:, :, None, :]
        sin = freqs[..., half:2 * half][:, :, None, :]
        x1 = u[..., :half]
        x2 = u[..., half:2 * half]
        out[..., :half] = x1 * cos - x2 * sin
        out[..., half:2 * half] = x2 * cos + x1 * sin
    return out


def pack_region_bitmap(ids, regions):
    """Membership words [..., ceil(regions / 32)] int32 of every id row.

    CSA page, ``pack_region_bitmap``: bit ``r % 32`` of word ``r // 32`` is set
    exactly when region ``r`` occurs in the row; ids at or above ``regions``
    are padding and repeated ids are allowed.  Negative ids are padding too
    (the route lists here pad with -1).  Words are returned as int32 bit
    patterns (bit 31 is the sign bit).
    """
    ids = np.asarray(ids)
    lead = ids.shape[:-1]
    words = (regions + 31) // 32
    flat = ids.reshape(-1, ids.shape[-1])
    out = np.zeros((flat.shape[0], words), dtype=np.uint32)
    for r in range(flat.shape[0]):
        for x in flat[r]:
            x = int(x)
            if 0 <= x < regions:
                out[r, x // 32] |= np.uint32(1) << np.uint32(x % 32)
    return out.view(np.int32).reshape(lead + (words,))


# ---------------------------------------------------------------------------
# a2: indexer scores
# ---------------------------------------------------------------------------

def indexer_scores(qI, w, kc, c, scale=None, cu_seqlens=None, row_lens=None, q0=0, q1=None,
                   row_chunk=256):
    """Scores [B, q1-q0, NB] (float64); invisible entries are -inf.

    ``s[t, j] = scale * sum_h w[t, h] * max(0, qI[t, h] . kc[j])`` over the
    blocks ``j`` of the query's own document with local index below
    ``nb(t) = floor((pos+1)/c)`` (QSA page, ``select_qsa_token_ids``: ReLU
    head sum over complete visible blocks, divided by sqrt(D); CSA page,
    ``indexer_score_tile``: signed FP32 head weights).  ``scale`` defaults
    to 1/sqrt(D_idx).  Padding queries score -inf everywhere.
    """
    qI = np.asarray(qI)
    w = np.asarray(w)
    kc = np.asarray(kc, dtype=np.float64)
    B, S, H, D = qI.shape
    q1 = S if q1 is None else q1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    NB = kc.shape[1]
    docs = documents(B, S, cu_seqlens, row_lens)
    valid, start, base, nb = token_info(docs, S, c)
    out = np.full((B, q1 - q0, NB), NEG_INF, dtype=np.float64)
    for b in range(B):
        for r0 in range(q0, q1, row_chunk):
            r1 = min(q1, r0 + row_chunk)
            qs = qI[b, r0:r1].astype(np.float64)                     # [t, H, D]
            ws = w[b, r0:r1].astype(np.float64)                      # [t, H]
            dots = qs @ kc[b].T                                      # [t, H, NB]
            s = scale * (ws[:, None, :] @ np.maximum(dots, 0.0))[:, 0, :]
            j = np.arange(NB)[None, :]
            lo = base[b, r0:r1, None]
            vis = valid[b, r0:r1, None] & (j >= lo) & (j < lo + nb[b, r0:r1, None])
            out[b, r0 - q0:r1 - q0] = np.where(vis, s, NEG_INF)
    return out


# ---------------------------------------------------------------------------
# a3: top-k block selection
# ---------------------------------------------------------------------------

def select_topk(scores, c, topk, cu_seqlens=None, row_lens=None, q0=0, S=None):
    """Selected global block IDs [B, rows, topk] (ascending, -1 suffix) and counts.

    The ``k_eff = min(topk, nb(t))`` highest visible scores win (QSA page,
    ``select_qsa_token_ids``: best ``budget / c`` blocks; CSA page,
    ``RegionMetadata.dense_region_ids``: with no more than ``topk`` visible
    regions all of them are taken).  Ties go to the lower block ID; -0.0 and
    +0.0 compare equal.  The chosen IDs are written in ascending order (CSA
    page, ``RegionSelection.region_ids`` is sorted) and the rest is -1.
    """
    scores = np.asarray(scores)
    B, rows, NB = scores.shape
    S = q0 + rows if S is None else S
    docs = documents(B, S, cu_seqlens, row_lens)
    valid, start, base, nb = token_info(docs, S, c)
    sel = np.full((B, rows, topk), -1, dtype=np.int32)
    cnt = np.zeros((B, rows), dtype=np.int32)
    for b in range(B):
        for r in range(rows):
            t = q0 + r
            if not valid[b, t] or nb[b, t] == 0:
                continue
            n, lo = int(nb[b, t]), int(base[b, t])
            k = min(topk, n)
            vis = scores[b, r, lo:lo + n]
            ids = np.arange(n)
            order = np.lexsort((ids, -vis))[:k]   # score descending, then ID ascending
            chosen = np.sort(order) + lo
            sel[b, r, :k] = chosen
            cnt[b, r] = k
    return sel, cnt


def near_tie_rows(scores, c, topk, cu_seqlens=None, row_lens=None, q0=0, S=None, rel=1e-4):
    """Rows whose k-th and (k+1)-th visible scores are within ``rel`` relative.

    Only sparse rows (``nb > topk``) can be near-ties.  Such rows are
    excluded from bit-exact route comparison and counted instead.
    """
    scores = np.asarray(scores)
    B, rows, NB = scores.shape
    S = q0 + rows if S is None else S
    docs = documents(B, S, cu_seqlens, row_lens)
    valid, start, base, nb = token_info(docs, S, c)
    out = np.zeros((B, rows), dtype=bool)
    for b in range(B):
        for r in range(rows):
            t = q0 + r
            n = int(nb[b, t])
            if not valid[b, t] or n <= topk:
                continue
            lo = int(base[b, t])
            v = np.sort(scores[b, r, lo:lo + n])[::-1]
            a, z = v[topk - 1], v[topk]
            out[b, r] = bool(a == z) or abs(a - z) <= rel * max(abs(a), abs(z))
    return out


# ---------------------------------------------------------------------------
# a4: route expansion and compaction
# ---------------------------------------------------------------------------

def route_width(topk, c, window):
    """Fixed route width ``topk*c + max(window, c-1)``.

    With no window this is the QSA page's ``budget + c - 1`` (indexer
    ``forward`` return shape); a window of W tokens can replace the tail.
    """
    return topk * c + max(window, c - 1)


def expand_routes(sel, cnt, c, window, topk, cu_seqlens=None, row_lens=None, L=None, rows=None):
    """Token routes [B, S, L] (ascending, unique, -1 suffix) and lengths [B, S].

    ``R(t)`` = tokens of the selected blocks, plus the tokens of the current
    incomplete group ``[doc_start + nb*c, t]`` (QSA page,
    ``select_qsa_token_ids``: 0..c-1 tail tokens), plus the window
    ``[max(doc_start, t-W+1), t]`` (CSA page, ``RegionMetadata.window_layout``:
    the window holds the query and at most W-1 earlier keys); duplicates
    removed (QSA page, ``qsa_gqa_attention``: duplicates collapse), sorted,
    padded with -1 (QSA page, ``QSARouteSelection.selected_token_ids``).
    ``rows`` optionally restricts the evaluation to a list of (b, t) pairs.
    """
    sel = np.asarray(sel)
    B, S, _ = sel.shape
    L = route_width(topk, c, window) if L is None else L
    docs = documents(B, S, cu_seqlens, row_lens)
    valid, start, base, nb = token_info(docs, S, c)
    routes = np.full((B, S, L), -1, dtype=np.int32)
    lens = np.zeros((B, S), dtype=np.int32)
    todo = [(b, t) for b in range(B) for t in range(S)] if rows is None else rows
    for b, t in todo:
            if not valid[b, t]:
                continue
            a = int(start[b, t])
            k = int(cnt[b, t])
            local = sel[b, t, :k].astype(np.int64) - int(base[b, t])
            parts = [(a + local[:, None] * c + np.arange(c)[None, :]).ravel()]
            parts.append(np.arange(a + int(nb[b, t]) * c, t + 1))
            if window > 0:
                parts.append(np.arange(max(a, t - window + 1), t + 1))
            r = np.unique(np.concatenate(parts))
            if len(r) > L:
                raise ValueError("route longer than its width")
            routes[b, t, :len(r)] = r
            lens[b, t] = len(r)
    return routes, lens


def compact_routes(ids, key_count):
    """Ascending unique valid prefix of arbitrary signed ID rows.

    Latent page, ``_compact_and_sort_indices``: negative entries are invalid;
    the result is an ascending valid prefix plus its length.  Entries at or
    beyond ``key_count`` are also dropped and counted (``n_out_of_range``).
    Input [..., W] -> (out [..., W] int32 with -1 suffix, len [...], n_out_of_range).
    """
    ids = np.asarray(ids)
    shape = ids.shape
    flat = ids.reshape(-1, shape[-1]).astype(np.int64)
    out = np.full(flat.shape, -1, dtype=np.int32)
    lens = np.zeros(flat.shape[0], dtype=np.int32)
    bad = 0
    for r in range(flat.shape[0]):
        row = flat[r]
        bad += int(np.count_nonzero(row >= key_count))
        u = np.unique(row[(row >= 0) & (row < key_count)])
        out[r, :len(u)] = u
        lens[r] = len(u)
    return out.reshape(shape), lens.reshape(shape[:-1]), bad


# ---------------------------------------------------------------------------
# a5: forward / reverse block lists
# ---------------------------------------------------------------------------

def block_lists(routes, lens, S_k, block_q, block_k, reverse=False, rows=None):
    """Block-sparse lists from token routes.

    Forward (FA4 page, ``_selected_block_lists``, ``_block_lists``): for
    every tile of ``block_q`` queries, the ascending key tiles of
    ``block_k`` keys holding at least one routed key of one of its queries.
    Reverse (``reverse=True``, used by backward): for every key tile, the
    ascending query tiles that reach it.  Returns counts [B, rows] and
    indices [B, rows, width] with -1 after the count; width is the number of
    tiles on the other axis.  ``rows`` (list of (b, row)) restricts which
    list rows are evaluated; the others keep count 0.
    """
    routes = np.asarray(routes)
    lens = np.asarray(lens)
    B, S_q, _ = routes.shape
    nqt = -(-S_q // block_q)
    nkt = -(-S_k // block_k)
    n_rows, width = (nkt, nqt) if reverse else (nqt, nkt)
    counts = np.zeros((B, n_rows), dtype=np.int32)
    indices = np.full((B, n_rows, width), -1, dtype=np.int32)
    if rows is not None:
        # one list row at a time, straight from its definition
        L = routes.shape[2]
        pos = np.arange(L)[None, :]
        for b, r in rows:
            if reverse:
                lo, hi = r * block_k, min((r + 1) * block_k, S_k)
                hit = np.zeros(S_q, dtype=bool)
                for t0 in range(0, S_q, 2048):        # row chunks keep temporaries small
                    rr = routes[b, t0:t0 + 2048]
                    live = pos < np.minimum(lens[b, t0:t0 + 2048], L)[:, None]
                    hit[t0:t0 + 2048] = np.any(live & (rr >= lo) & (rr < hi), axis=1)
                nz = np.unique(np.nonzero(hit)[0] // block_q)
            else:
                t0, t1 = r * block_q, min((r + 1) * block_q, S_q)
                live = pos < np.minimum(lens[b, t0:t1], L)[:, None]
                ids = routes[b, t0:t1][live]
                nz = np.unique(ids[(ids >= 0) & (ids < S_k)] // block_k)
            counts[b, r] = len(nz)
            indices[b, r, :len(nz)] = nz
        return counts, indices
    for b in range(B):
        grid = np.zeros((nqt, nkt), dtype=bool)
        for t in range(S_q):
            n = int(lens[b, t])
            if n:
                grid[t // block_q, routes[b, t, :n] // block_k] = True
        if reverse:
            grid = grid.T
        for r in range(n_rows):
            nz = np.nonzero(grid[r])[0]
            counts[b, r] = len(nz)
            indices[b, r, :len(nz)] = nz
    return counts, indices


def split_full_blocks(routes, lens, S_k, block_q, block_k, counts, indices, reverse=False):
    """Split block lists into full and partial blocks.

    FA4 page, ``_split_forward_full_blocks`` / ``_split_backward_full_blocks``
    (with ``_BackwardBlockPartition``): the blocks of a forward list (key
    tiles per query tile) or a reverse list (query tiles per key tile) are
    separated into "full" blocks, which need no mask, and "partial" ones,
    keeping each list's order.  A block (query tile i, key tile j) is full
    when every pair of its rectangle ``[i*block_q, min((i+1)*block_q, S_q))
    x [j*block_k, min((j+1)*block_k, S_k))`` is routed (the key lies in the
    query's route); the page establishes this for complete causal
    rectangles of an all-selected query prefix, which is one case of it.
    Returns (full_counts, full_indices, part_counts, part_indices) in the
    layout of ``counts`` / ``indices`` (-1 after each count).
    """
    routes = np.asarray(routes)
    lens = np.asarray(lens)
    counts = np.asarray(counts)
    indices = np.asarray(indices)
    B, S_q, _ = routes.shape
    full_c = np.zeros_like(counts)
    part_c = np.zeros_like(counts)
    full_i = np.full_like(indices, -1)
    part_i = np.full_like(indices, -1)
    for b in range(B):
        routed = np.zeros((S_q, S_k), dtype=bool)       # the dense (query, key) mask of the routes
        for t in range(S_q):
            ids = routes[b, t, :max(0, int(lens[b, t]))]
            routed[t, ids[(ids >= 0) & (ids < S_k)]] = True
        for r in range(counts.shape[1]):
            for e in range(int(counts[b, r])):
                o = int(indices[b, r, e])
                i, j = (o, r) if reverse else (r, o)
                rect = routed[i * block_q:min((i + 1) * block_q, S_q), j * block_k:min((j + 1) * block_k, S_k)]
                if rect.size and rect.all():
                    full_i[b, r, full_c[b, r]] = o
                    full_c[b, r] += 1
                else:
                    part_i[b, r, part_c[b, r]] = o
                    part_c[b, r] += 1
    return full_c, full_i, part_c, part_i


# ---------------------------------------------------------------------------
# a6 / a7: sparse GQA attention over gathered keys
# ---------------------------------------------------------------------------

def _route_set(row, S_k):
    row = np.asarray(row, dtype=np.int64)
    return np.unique(row[(row >= 0) & (row < S_k)])


def attention_fwd(q, k, v, routes, scale=None, rows=None):
    """Sparse GQA forward: output [B, S_q, Hq, Dv] and lse [B, Hq, S_q] (float64).

    QSA page, ``gathered_qsa_gqa_attention``: each query attends only to the
    keys and values at its route IDs; query head ``h`` uses KV group
    ``h // (Hq/Hkv)`` (grouped query layout [B, Q, Hkv, G, D]); -1 and
    out-of-range slots are ignored and repeated IDs count once; the score
    multiplier defaults to 1/sqrt(D).  ``o = softmax(scale q K_R^T) V_R``.
    A query with an empty route gets o = 0 and lse = -inf.  ``rows``
    optionally restricts the evaluation to a list of (b, t) pairs.
    """
    # inputs stay in their own dtype; each gathered piece is widened to float64
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, S_q, Hq, D = q.shape
    S_k, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = np.zeros((B, S_q, Hq, Dv), dtype=np.float64)
    lse = np.full((B, Hq, S_q), NEG_INF, dtype=np.float64)
    todo = [(b, t) for b in range(B) for t in range(S_q)] if rows is None else rows
    for b, t in todo:
        ids = _route_set(routes[b, t], S_k)
        if len(ids) == 0:
            continue
        kg = k[b, ids].astype(np.float64).transpose(1, 0, 2)    # [Hkv, n, D]
        vg = v[b, ids].astype(np.float64).transpose(1, 0, 2)    # [Hkv, n, Dv]
        qg = q[b, t].astype(np.float64).reshape(Hkv, G, D)
        x = scale * (qg @ kg.transpose(0, 2, 1))                # [Hkv, G, n]
        m = x.max(axis=-1, keepdims=True)
        ls = m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True))
        p = np.exp(x - ls)
        o[b, t] = (p @ vg).reshape(Hq, Dv)
        lse[b, :, t] = ls.reshape(Hq)
    return o, lse


def attention_bwd(q, k, v, routes, dO, scale=None, rows=None, keys=None):
    """Sparse GQA backward: dq, dk, dv (float64) for dO.

    Gradients of the forward above with respect to q, k and v (QSA page,
    ``gathered_qsa_gqa_attention`` is differentiable; the indexer is frozen,
    so routes carry no gradient).  Per query and head:
    ``P = softmax(x)``, ``dP = dO V_R^T``, ``dS = P (dP - rowsum(dO * o))``,
    ``dq = scale dS K_R``, ``dK_R += scale dS^T q``, ``dV_R += P^T dO``;
    the key/value sums run over every query that routes to that key.
    ``rows`` (list of (b, t)) restricts the dq evaluation and ``keys`` (list
    of (b, key)) the dk/dv evaluation; other entries are left at zero.  With
    either given, only the queries they need are evaluated.
    """
    # inputs stay in their own dtype; each gathered piece is widened to float64
    q, k, v, dO = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(dO)
    B, S_q, Hq, D = q.shape
    S_k, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    restricted = rows is not None or keys is not None
    want_rows = set(map(tuple, rows)) if rows is not None else set()
    key_sets = {}
    if keys is not None:
        for b_, kk in keys:
            key_sets.setdefault(int(b_), set()).add(int(kk))
    for b in range(B):
        ks = np.array(sorted(key_sets.get(b, ())), dtype=np.int64)
        for t in range(S_q):
            ids = _route_set(routes[b, t], S_k)
            if len(ids) == 0:
                continue
            need_q = (not restricted) or (b, t) in want_rows
            hit = np.isin(ids, ks) if keys is not None else None
            need_k = (not restricted) or (hit is not None and hit.any())
            if not (need_q or need_k):
                continue
            kg = k[b, ids].astype(np.float64).transpose(1, 0, 2)    # [Hkv, n, D]
            vg = v[b, ids].astype(np.float64).transpose(1, 0, 2)    # [Hkv, n, Dv]
            qg = q[b, t].astype(np.float64).reshape(Hkv, G, D)
            dog = dO[b, t].astype(np.float64).reshape(Hkv, G, Dv)
            x = scale * (qg @ kg.transpose(0, 2, 1))    # [Hkv, G, n]
            m = x.max(axis=-1, keepdims=True)
            p = np.exp(x - m)
            p /= p.sum(axis=-1, keepdims=True)
            og = p @ vg                                 # [Hkv, G, Dv]
            delta = np.sum(dog * og, axis=-1, keepdims=True)
            dp = dog @ vg.transpose(0, 2, 1)            # [Hkv, G, n]
            ds = p * (dp - delta)
            if need_q:
                dq[b, t] = (scale * (ds @ kg)).reshape(Hq, D)
            if need_k:
                sel = slice(None) if hit is None else hit
                # ids are unique, so the fancy-indexed += adds each key once
                dk[b, ids[sel]] += scale * (ds[:, :, sel].transpose(0, 2, 1) @ qg).transpose(1, 0, 2)
                dv[b, ids[sel]] += (p[:, :, sel].transpose(0, 2, 1) @ dog).transpose(1, 0, 2)
    return dq, dk, dv


def latent_attention_fwd(q, kv, idx, scale, dv=512):
    """Latent single-KV-head sparse attention forward (latent page, ``cudnn_sparse_attention``).

    q [T, H, Dqk], shared latent kv [T, 1, Dqk], index lists [T, 1, W]
    (-1 invalid); keys are the full latent rows, values their first ``dv``
    channels.  Returns o [T, H, dv] and lse [H, T].
    """
    k = np.asarray(kv)[None]
    o, lse = attention_fwd(np.asarray(q)[None], k, k[..., :dv], np.asarray(idx)[None, :, 0, :], scale)
    return o[0], lse[0]


def latent_attention_bwd(q, kv, idx, dO, scale, dv=512, rows=None, keys=None):
    """Latent backward: dq [T, H, Dqk] and the merged latent gradient dkv [T, 1, Dqk].

    Keys and values are views of one latent tensor, so its gradient is
    ``dK + [dV, 0]`` (the value part covers the first ``dv`` channels).
    ``rows`` / ``keys`` (lists of token indices) restrict the evaluation as
    in ``attention_bwd``.
    """
    k = np.asarray(kv)[None]
    rows = None if rows is None else [(0, int(t)) for t in rows]
    keys = None if keys is None else [(0, int(j)) for j in keys]
    dq, dk, dvv = attention_bwd(np.asarray(q)[None], k, k[..., :dv], np.asarray(idx)[None, :, 0, :],
                                np.asarray(dO)[None], scale, rows=rows, keys=keys)
    dkv = dk[0].copy()
    dkv[..., :dv] += dvv[0]
    return dq[0], dkv


# ---------------------------------------------------------------------------
# per-KV-group routes (CSA page: scores and selections [batch, groups, ...])
# ---------------------------------------------------------------------------

def indexer_scores_grouped(qI, w, kc, c, scale=None, cu_seqlens=None, row_lens=None, q0=0, q1=None):
    """Scores of every KV group [R, B, q1-q0, NB] (float64); invisible entries are -inf.

    CSA page, ``indexer_score_tile``: the index queries carry a group axis
    ([batch, queries, groups, heads, dim], signed weights [batch, queries,
    groups, heads]) and every group gets its own score row over the shared
    region summaries:
    ``s[g, b, t, j] = scale * sum_h w[b,t,g,h] * max(0, qI[b,t,g,h] . kc[b,j])``,
    with the visibility of ``indexer_scores``.  ``scale`` defaults to
    1/sqrt(D_idx).  The group axis leads the result so that each group's
    scores are one contiguous [B, rows, NB] block.
    """
    qI = np.asarray(qI)
    w = np.asarray(w)
    R = qI.shape[2]
    return np.stack([indexer_scores(qI[:, :, g], w[:, :, g], kc, c, scale, cu_seqlens, row_lens, q0, q1)
                     for g in range(R)])


def _group_of_heads(Hq, Hkv, R):
    """Route group of every query head: head h reads KV head h // (Hq/Hkv);
    with R == Hkv route groups that KV head's group, with R == 1 the shared one."""
    if R not in (1, Hkv):
        raise ValueError("route groups must be 1 or the number of KV heads")
    G = Hq // Hkv
    return [(h // G) if R > 1 else 0 for h in range(Hq)]


def attention_fwd_grouped(q, k, v, routes, scale=None, rows=None):
    """Sparse GQA forward with per-KV-group routes [R, B, S_q, L] (R = 1 or Hkv).

    CSA page, ``pack_region_bitmap`` / ``indexer_score_tile``: selections
    carry a groups axis, one route per (batch, KV group, query); FA4 page,
    ``_provider_heads``: a group's route serves the consecutive query heads
    sharing that KV head.  Every KV group is the forward of ``attention_fwd``
    over its own heads and its own route; R == 1 is ``attention_fwd``.
    Output [B, S_q, Hq, Dv] and lse [B, Hq, S_q] (float64).
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    routes = np.asarray(routes)
    R = routes.shape[0]
    Hq, Hkv = q.shape[2], k.shape[2]
    _group_of_heads(Hq, Hkv, R)
    if R == 1:
        return attention_fwd(q, k, v, routes[0], scale, rows)
    G = Hq // Hkv
    o = np.zeros(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.full((q.shape[0], Hq, q.shape[1]), NEG_INF, dtype=np.float64)
    for g in range(R):
        hs = slice(g * G, (g + 1) * G)
        og, lg = attention_fwd(q[:, :, hs], k[:, :, g:g + 1], v[:, :, g:g + 1], routes[g], scale, rows)
        o[:, :, hs] = og
        lse[:, hs] = lg
    return o, lse


def attention_bwd_grouped(q, k, v, routes, dO, scale=None, rows=None, keys=None):
    """Gradients dq, dk, dv (float64) of ``attention_fwd_grouped`` for dO.

    Per KV group the gradient of ``attention_bwd`` over that group's heads
    and route (a key's dk/dv in group g sums over the queries whose group-g
    route holds it); R == 1 is ``attention_bwd``.  ``rows`` / ``keys``
    restrict the evaluation as there.
    """
    q, k, v, dO = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(dO)
    routes = np.asarray(routes)
    R = routes.shape[0]
    Hq, Hkv = q.shape[2], k.shape[2]
    _group_of_heads(Hq, Hkv, R)
    if R == 1:
        return attention_bwd(q, k, v, routes[0], dO, scale, rows, keys)
    G = Hq // Hkv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for g in range(R):
        hs = slice(g * G, (g + 1) * G)
        a, b_, c_ = attention_bwd(q[:, :, hs], k[:, :, g:g + 1], v[:, :, g:g + 1], routes[g], dO[:, :, hs],
                                  scale, rows, keys)
        dq[:, :, hs] = a
        dk[:, :, g:g + 1] = b_
        dv[:, :, g:g + 1] = c_
    return dq, dk, dv


# ---------------------------------------------------------------------------
# whole route pipeline
# ---------------------------------------------------------------------------

def route_pipeline(kI, qI, w, gamma, freqs, c, topk, window, eps=1e-5, scale=None,
                   cu_seqlens=None, row_lens=None):
    """compress -> score -> select -> expand, as the QSA indexer composes them."""
    kc, cu_blocks = compress_keys(kI, gamma, eps, freqs, c, cu_seqlens, row_lens)
    s = indexer_scores(qI, w, kc, c, scale, cu_seqlens, row_lens)
    sel, cnt = select_topk(s, c, topk, cu_seqlens, row_lens)
    routes, lens = expand_routes(sel, cnt, c, window, topk, cu_seqlens, row_lens)
    return dict(kc=kc, cu_blocks=cu_blocks, scores=s, sel=sel, cnt=cnt, routes=routes, lens=lens)


# ---------------------------------------------------------------------------
# CSA variant: region payload gather, learned region summaries, E4M3
# rounding, selection with the current-region slot
# ---------------------------------------------------------------------------

def _round_to_grid(x, mant_bits, min_exp):
    """Round-to-nearest-even onto a binary floating-point grid with
    ``mant_bits`` stored mantissa bits and smallest normal exponent ``min_exp``
    (below it the grid is uniform: subnormals), unbounded above."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(np.where(fin, x, 1.0))          # |x| = m 2^e, 0.5 <= m < 1: leading bit 2^(e-1)
    step = np.ldexp(1.0, np.maximum(e - 1, min_exp) - mant_bits)
    out[fin] = (np.rint(x / step) * step)[fin]      # np.rint rounds halves to even
    return out


def round_to_bf16(x):
    """bfloat16 round-to-nearest-even (8 significand bits, float32's exponent range), as float64."""
    q = _round_to_grid(x, 7, -126)
    return np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, q), q)


def round_to_e4m3(x):
    """E4M3 (OCP FN: 4 exponent bits with bias 7, 3 mantissa bits, no infinities)
    round-to-nearest-even, as float64 -- the CSA page's "E4M3-rounded"
    tensors (index queries and region summaries) are BF16 tensors holding
    such values.  The largest finite value is 448; a value that rounds past
    it (to 480 on the grid) or is not finite becomes NaN, as torch's
    float8_e4m3fn conversion does.  Zero keeps its sign."""
    x = np.asarray(x, dtype=np.float64)
    q = _round_to_grid(x, 3, -6)
    return np.where(np.isfinite(q) & (np.abs(q) <= 448.0), q, np.nan)


def gather_region_payload(keys, logits, sources, valid):
    """CSA page, ``gather_region_payload`` / ``_gather_region_payload``: the
    index keys and compression logits of every region's source tokens,
    gathered without arithmetic into [B, R, region_size, D].

    ``keys``, ``logits`` [B, T, D]; ``sources`` int32 [B, R, region_size]
    (token index, -1 for a missing slot); ``valid`` bool of the same shape
    (excludes padding tokens and missing slots).  Reading: slots that are not
    valid hold zeros (the page leaves their content open; the summary
    ignores them).
    """
    keys = np.asarray(keys)
    logits = np.asarray(logits)
    src = np.asarray(sources).astype(np.int64)
    ok = np.asarray(valid, dtype=bool) & (src >= 0) & (src < keys.shape[1])
    idx = np.where(ok, src, 0)
    b = np.arange(keys.shape[0])[:, None, None]
    pk = np.where(ok[..., None], keys[b, idx], 0).astype(keys.dtype)
    pz = np.where(ok[..., None], logits[b, idx], 0).astype(logits.dtype)
    return pk, pz


def summarize_region_payload(pk, pz, valid, fp32_only=False):
    """CSA page, ``_summarize_region_payload`` (reading; the page states FP32
    arithmetic and two quantisation roundings, not the formula).

    Per region r and dimension d, the compression logits of the region's
    valid slots weight their keys through a softmax over the slots
    (``Step5SparseIndexer.project_keys``: per-dimension compression logits):

        s[r, d] = sum_s exp(z[r,s,d] - m[r,d]) k[r,s,d] / sum_s exp(z[r,s,d] - m[r,d]),
        m[r, d] = max over valid slots s of z[r,s,d],

    evaluated in float32, then rounded to BF16 and that value to E4M3
    (``indexer_score_tile`` takes E4M3-rounded BF16 summaries).  A region with
    no valid slot summarises to 0.  ``fp32_only`` returns the float32 values
    before the two roundings (to locate rounding boundaries).
    """
    k = np.asarray(pk, dtype=np.float32)
    z = np.asarray(pz, dtype=np.float32)
    ok = np.asarray(valid, dtype=bool)[..., None]
    zm = np.where(ok, z, np.float32(-np.inf))
    m = np.max(zm, axis=-2, keepdims=True)
    any_ok = np.isfinite(m)
    m = np.where(any_ok, m, np.float32(0.0))
    e = np.where(ok, np.exp(zm - m, dtype=np.float32), np.float32(0.0))
    den = np.sum(e, axis=-2, dtype=np.float32)
    num = np.sum(e * k, axis=-2, dtype=np.float32)
    s = np.where(den > 0, num / np.where(den > 0, den, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    if fp32_only:
        return s
    return round_to_e4m3(round_to_bf16(s))


def region_bases(docs, c: int):
    """Global region ID of every document's first region when every token
    belongs to a region (CSA page, ``region_metadata``: regions of
    ``region_size`` tokens, reset at every document boundary, so a
    document of ``len`` tokens has ``ceil(len / c)`` regions, the last one
    possibly incomplete), and the total region count of each row."""
    out, totals = [], []
    for row in docs:
        base, bases = 0, []
        for (a, e) in row:
            bases.append(base)
            base += -(-(e - a) // c)
        out.append(bases)
        totals.append(base)
    return out, totals


def select_regions_csa(scores, c, topk, cu_seqlens=None, row_lens=None, q0=0, S=None):
    """CSA page, ``RegionSelection.region_ids`` with ``RegionMetadata.current``
    (reading): ids [B, rows, topk + 1] int32 and their counts [B, rows].

    A query at document position ``pos`` lies in region ``floor(pos / c)`` of
    its document, the current region, which it always keeps.  Its historical
    regions are the ones before that, ``floor(pos / c)`` of them (all
    complete); they compete for ``topk`` slots by score as in
    ``select_topk`` (ties to the lower index; with at most ``topk`` of them
    all are taken).  ``scores`` are the block scores of this library's
    numbering (complete blocks only, as written by ``indexer_scores``); the
    output uses the page's numbering, in which every document's regions
    (incomplete last one included) are consecutive, sorted ascending, with
    the unused slots holding the sentinel R = the row's region count.
    Padding queries hold only sentinels (count 0).
    """
    scores = np.asarray(scores)
    B, rows, NB = scores.shape
    S = q0 + rows if S is None else S
    docs = documents(B, S, cu_seqlens, row_lens)
    valid, start, base, nb = token_info(docs, S, c)
    rbases, totals = region_bases(docs, c)
    ids = np.zeros((B, rows, topk + 1), dtype=np.int32)
    cnt = np.zeros((B, rows), dtype=np.int32)
    for b in range(B):
        ids[b] = totals[b]
        dstarts = [a for (a, e) in docs[b]]
        for r in range(rows):
            t = q0 + r
            if not valid[b, t]:
                continue
            d = dstarts.index(int(start[b, t]))
            pos = t - int(start[b, t])
            h = pos // c                          # historical regions = complete blocks before the current one
            k = min(topk, h)
            lo = int(base[b, t])
            if k > 0:
                vis = scores[b, r, lo:lo + h]
                order = np.lexsort((np.arange(h), -vis))[:k]
                chosen = np.sort(order)
            else:
                chosen = np.zeros(0, dtype=np.int64)
            rb = rbases[b][d]
            ids[b, r, :k] = rb + chosen
            ids[b, r, k] = rb + h
            cnt[b, r] = k + 1
    return ids, cnt
