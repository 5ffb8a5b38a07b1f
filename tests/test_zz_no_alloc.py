"""The allocation-free fused route call against the workspace call, through the C ABI.

irb_route_topk_fused_noalloc runs the same kernels as irb_route_topk_fused on
the library's static per-device scratch; its selections must equal the
workspace call's bit for bit.  Two calls in a row, the second on a smaller
input, so that the second reads a scratch the first left filled.
"""
import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import synth
from gpu_util import act_dtype, banner, to_dev

pytestmark = pytest.mark.gpu


def _inputs(S, layout):
    wl = synth.WORKLOADS["s8192" if layout == "single" else "varlen"]
    cu = None
    if layout == "packed":
        cu, _ = synth.varlen_documents(np.random.default_rng(S), S, min_len=16, max_len=S // 3, max_pad=S // 8)
    x = synth.make_inputs(wl, parts=("route",), S=S, cu_seqlens=cu)
    dt = act_dtype(wl.dtype)
    d = dict(kI=to_dev(x["kI"], dt), qI=to_dev(x["qI"], dt), w=to_dev(x["w"]), gamma=to_dev(x["gamma"]),
             freqs=to_dev(x["freqs"]), cu=to_dev(x["cu_seqlens"]))
    return wl, d


@pytest.mark.parametrize("S,layout,topk", [(8192, "single", 512), (4096, "packed", 64)])
def test_noalloc_route_equals_workspace_route(S, layout, topk):
    banner(f"no-alloc fused route S={S} {layout} topk={topk}")
    wl, d = _inputs(S, layout)
    kc, cub = irb.compress_keys(d["kI"], d["gamma"], d["freqs"], wl.c, 1e-5, d["cu"])
    sel_a, cnt_a = irb.route_topk_fused(d["qI"], d["w"], kc, wl.c, topk, cu_blocks=cub, cu_seqlens=d["cu"])
    # outputs pre-filled with garbage: every row must be written
    sel_b = torch.full_like(sel_a, 12345)
    cnt_b = torch.full_like(cnt_a, -7)
    irb.route_topk_fused_noalloc(d["qI"], d["w"], kc, wl.c, topk, cu_blocks=cub, cu_seqlens=d["cu"], sel=sel_b,
                                 cnt=cnt_b)
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b)
    assert torch.equal(sel_a, sel_b)
    # the same call again on a smaller input (a prefix of the sequence): the
    # scratch still holds the first call's split keys and scores
    S2 = S // 4
    wl2, d2 = _inputs(S2, "single")
    kc2, _ = irb.compress_keys(d2["kI"], d2["gamma"], d2["freqs"], wl2.c, 1e-5)
    t2 = min(topk, S2 // wl2.c // 4)
    sel_c, cnt_c = irb.route_topk_fused(d2["qI"], d2["w"], kc2, wl2.c, t2)
    sel_d, cnt_d = irb.route_topk_fused_noalloc(d2["qI"], d2["w"], kc2, wl2.c, t2)
    torch.cuda.synchronize()
    assert torch.equal(cnt_c, cnt_d)
    assert torch.equal(sel_c, sel_d)
    print(f"  rows {S} and {S2}: selections identical; sparse rows {int((cnt_a == topk).sum())}")
