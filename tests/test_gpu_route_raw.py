"""Index-query preparation fused into the route call (irb_route_topk_fused_raw)
against the FP64 oracle, through the C ABI.

The fused call normalises and rotates the raw index queries inside the score
kernel.  Two checks per case:

* against the two-call path (irb_prepare_index_queries, then
  irb_route_topk_fused) the selection must be identical, bit for bit: the
  score kernel repeats the preparation's FP32 arithmetic step for step;
* against the oracle: its FP64 prepared queries, rounded to bf16 (round to
  nearest even) for bf16 inputs, are scored and selected.  Rows that agree are
  compared bit for bit (selection, routes, lengths).  A row that differs must
  still be a correct top-k: some perturbation of each score within the FP32
  scoring bound plus the preparation's own rounding ambiguity makes the GPU's
  set the top k.  The ambiguity: an element whose FP64 value lies within the
  FP32 error E of a bf16 rounding boundary may round either way, moving a
  score by at most scale * sum_h |w_h| * sum_d |q'_hd - q_hd| * |k_d| (ReLU is
  1-Lipschitz); FP32 queries are not rounded and move by 2E.
"""
import math

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import act_dtype, banner, check_selection, host, prep_term_bound, rne_bf16, to_dev

pytestmark = pytest.mark.gpu


def _layout_case(name, S):
    if name == "single":
        return None, None, 1
    if name == "rows":
        return None, np.array([S, S // 3 + 5, 0], dtype=np.int32), 3
    if name == "packed":
        rng = np.random.default_rng(S)
        cu, _ = synth.varlen_documents(rng, S, min_len=16, max_len=max(32, S // 3), max_pad=min(511, S // 8))
        return cu, None, 1
    raise ValueError(name)


# (workload, S, layout, rotary width: None = the workload's D_idx)
CASES = [("s8192", 8192, "single", None), ("tiny", 512, "single", None), ("varlen", 4096, "packed", None),
         ("long", 4096, "single", 64), ("s8192", 1500, "rows", 0), ("tiny", 200, "rows", 0)]


@pytest.mark.parametrize("wl_name,S,layout,d_rope", CASES)
def test_route_raw_matches_two_calls_and_oracle(wl_name, S, layout, d_rope):
    wl = synth.WORKLOADS[wl_name]
    R = wl.D_idx if d_rope is None else d_rope
    banner(f"route raw {wl_name} S={S} {layout} D_rope={R}")
    cu, rl, B = _layout_case(layout, S)
    x = synth.make_inputs(wl, parts=("route",), S=S, B=B, cu_seqlens=cu, row_lens=rl)
    qfreqs = x["freqs"] if R == wl.D_idx else (synth.rope_table(synth.doc_positions(B, S, cu, rl), R) if R
                                              else np.zeros((B, S, 0), np.float32))
    dt = act_dtype(wl.dtype)
    q_raw = to_dev(x["qI"], dt)
    w, gamma = to_dev(x["w"]), to_dev(x["gamma"])
    fr = to_dev(qfreqs) if R else None
    dcu, drl = to_dev(cu), to_dev(rl)
    kc, cu_blocks = irb.compress_keys(to_dev(x["kI"], dt), gamma, to_dev(x["freqs"]), wl.c, 1e-5, dcu, drl)
    topk = min(wl.topk, max(4, S // wl.c // 4))
    sel, cnt = irb.route_topk_fused_raw(q_raw, gamma, fr, w, kc, wl.c, topk, cu_blocks=cu_blocks, cu_seqlens=dcu,
                                        row_lens=drl)
    # the two-call path: prepared queries materialised, then the same route call
    qp = irb.prepare_index_queries(q_raw, gamma, fr, 1e-5)
    sel2, cnt2 = irb.route_topk_fused(qp, w, kc, wl.c, topk, cu_blocks=cu_blocks, cu_seqlens=dcu, row_lens=drl)
    assert torch.equal(cnt, cnt2) and torch.equal(sel, sel2), "fused preparation differs from the two-call path"
    routes, lens = irb.expand_and_compact_routes(sel, cnt, wl.c, wl.window, topk, cu_blocks=cu_blocks,
                                                 cu_seqlens=dcu, row_lens=drl)

    # oracle: FP64 preparation, rounded as the GPU stores it, then scores and selection
    q64 = x["qI"].astype(np.float64)
    p64 = oracle.prepare_index_queries(q64, x["gamma"], qfreqs, 1e-5, d_rope=R)
    E = prep_term_bound(q64, x["gamma"], qfreqs, R)
    if dt == torch.bfloat16:
        qref = rne_bf16(p64)
        amb = rne_bf16(p64 + E) - rne_bf16(p64 - E)     # 0 where the rounding is decided
    else:
        qref, amb = p64, 2.0 * E
    print(f"  prepared elements with an undecided rounding: {int(np.count_nonzero(amb))} of {amb.size}")
    kc_h, _ = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, cu, rl)
    scale = 1.0 / math.sqrt(wl.D_idx)
    s_all = oracle.indexer_scores(qref, x["w"], kc_h, wl.c, scale, cu, rl)
    rsel, rcnt = oracle.select_topk(s_all, wl.c, topk, cu, rl)
    rr, rlens = oracle.expand_routes(rsel, rcnt, wl.c, wl.window, topk, cu, rl)
    ties = oracle.near_tie_rows(s_all, wl.c, topk, cu, rl)
    absk = np.abs(kc_h)

    def extra(b, t):
        dq = np.abs(amb[b, t])                           # [H, D]
        return scale * (np.abs(x["w"][b, t]) @ (dq @ absk[b].T))

    got = {"sel": host(sel)[None], "cnt": host(cnt)[None], "routes": host(routes)[None], "lens": host(lens)[None]}
    want = {"sel": rsel[None], "cnt": rcnt[None], "routes": rr[None], "lens": rlens[None], "ties": ties[None]}
    xr = dict(x, qI=qref)
    check_selection(wl, xr, topk, got, want, kc_h, grouped=False, extra=extra)
