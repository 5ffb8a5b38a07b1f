"""GPU parity of the Step-5 CSA variant (CSA page, step5.sparse) against the
FP64/FP32 oracle, through the C ABI: E4M3 rounding and the region payload
gather bit for bit, region summaries up to FP32 evaluation-order effects at
rounding boundaries, the selection with the current-region slot bit for bit
on fixed scores, and the composed CSA route pipeline."""
import math

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import DEV, SCORE_ERR, banner, host, score_bound, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_round_e4m3_bit_exact(dtype):
    banner(f"csa round_e4m3 {dtype}")
    rng = np.random.default_rng(21)
    x = rng.standard_normal(300000) * np.exp(rng.uniform(-14, 7, 300000))
    pos = np.unique(oracle.round_to_e4m3(np.abs(x)))
    pos = pos[np.isfinite(pos)]
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([x, mids, -mids, [463.99, 464.0, 465.0, 1e9, np.inf, -np.inf, np.nan, 0.0, -0.0, 2.0 ** -10]])
    xt = torch.from_numpy(x.astype(np.float32)).to(DEV).to(dtype)
    got = host(irb.round_e4m3(xt)).astype(np.float64)
    want = oracle.round_to_e4m3(xt.float().cpu().numpy().astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), f"{int((~same).sum())} differ, e.g. x={xt.float().cpu().numpy()[~same][:5]}"
    assert np.array_equal(np.signbit(got[want == 0]), np.signbit(want[want == 0]))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64), (torch.bfloat16, 8)])
def test_gather_region_payload_bit_exact(dtype, D):
    banner(f"csa gather {dtype} D={D}")
    rng = np.random.default_rng(D)
    B, T, R, rs = 2, 300, 77, 8
    keys = rng.standard_normal((B, T, D)).astype(np.float32)
    logits = rng.standard_normal((B, T, D)).astype(np.float32)
    src = rng.integers(-1, T + 5, (B, R, rs)).astype(np.int32)          # some ids past T count as missing
    valid = (src >= 0) & (rng.random((B, R, rs)) < 0.85)
    if dtype == torch.bfloat16:
        # the inputs are bf16 values on both sides (rounded on the host)
        keys, logits = oracle.round_to_bf16(keys), oracle.round_to_bf16(logits)
    k_d, z_d = to_dev(keys, dtype), to_dev(logits, dtype)
    pk, pz = irb.gather_region_payload(k_d, z_d, to_dev(src), to_dev(valid))
    rk, rz = oracle.gather_region_payload(keys, logits, src, valid & (src < T))
    np.testing.assert_array_equal(host(pk), rk)
    np.testing.assert_array_equal(host(pz), rz)


def _check_summaries(got, pk, pz, valid):
    """Equal to the oracle's E4M3 summaries, except where the float32 sum lies
    within 2^-20 (relative) of a BF16 rounding boundary: there the evaluation
    order (slot-sequential here, pairwise in NumPy) and exp's last bit may
    decide the boundary either way, so either side's rounding is accepted."""
    want = oracle.summarize_region_payload(pk, pz, valid)
    s32 = oracle.summarize_region_payload(pk, pz, valid, fp32_only=True).astype(np.float64)
    lo = oracle.round_to_e4m3(oracle.round_to_bf16(s32 * (1 - 2.0 ** -20)))
    hi = oracle.round_to_e4m3(oracle.round_to_bf16(s32 * (1 + 2.0 ** -20)))
    exact = got == want
    ok = exact | (got == lo) | (got == hi)
    assert ok.all(), f"{int((~ok).sum())} summaries differ beyond rounding boundaries"
    print(f"  summaries: {int((~exact).sum())} of {got.size} take the other side of a rounding boundary")


@pytest.mark.parametrize("dtype,rs,D", [(torch.bfloat16, 4, 128), (torch.float32, 16, 64), (torch.bfloat16, 1, 32)])
def test_summarize_region_payload(dtype, rs, D):
    banner(f"csa summarize {dtype} rs={rs} D={D}")
    rng = np.random.default_rng(rs * D)
    B, R = 2, 500
    pk = rng.standard_normal((B, R, rs, D)).astype(np.float32)
    pz = (2 * rng.standard_normal((B, R, rs, D))).astype(np.float32)
    valid = rng.random((B, R, rs)) < 0.8
    valid[0, 3] = False                                                 # an empty region
    pk_d, pz_d = to_dev(pk, dtype), to_dev(pz, dtype)
    got = host(irb.summarize_region_payload(pk_d, pz_d, to_dev(valid))).astype(np.float64)
    _check_summaries(got, host(pk_d), host(pz_d), valid)
    assert not got[0, 3].any()


@pytest.mark.parametrize("layout,topk,c,S,ties", [("single", 4, 4, 512, True), ("single", 64, 4, 4096, False),
                                                 ("packed", 8, 4, 2048, True), ("rows", 5, 3, 300, True)])
def test_select_regions_csa_bit_exact(layout, topk, c, S, ties):
    banner(f"csa select {layout} topk={topk} c={c} S={S}")
    rng = np.random.default_rng(S + topk)
    cu, rl, B = None, None, 1
    if layout == "packed":
        cu, _ = synth.varlen_documents(rng, S, min_len=5, max_len=S // 3, max_pad=S // 8)
    if layout == "rows":
        rl, B = np.array([S, S // 3 + 5, 0], dtype=np.int32), 3
    nb = S // c
    s = rng.standard_normal((B, S, nb))
    if ties:
        s = np.round(s * 2) / 2
    s = s.astype(np.float32)
    cub = None
    if cu is not None:
        cub = to_dev(np.concatenate([[0], np.cumsum(np.diff(cu) // c)]).astype(np.int32))
    ids, cnt = irb.select_regions_csa(to_dev(s), c, topk, S, cu_blocks=cub, cu_seqlens=to_dev(cu), row_lens=to_dev(rl))
    rids, rcnt = oracle.select_regions_csa(s.astype(np.float64), c, topk, cu, rl)
    np.testing.assert_array_equal(host(cnt), rcnt)
    np.testing.assert_array_equal(host(ids), rids)


def test_csa_route_pipeline():
    """Raw keys and compression logits -> gathered payload -> E4M3 summaries;
    E4M3-rounded index queries scored against them (irb_indexer_score_tile);
    selection with the current-region slot.  Regions are the complete groups
    of c consecutive tokens of one document (region_sources = their tokens)."""
    banner("csa pipeline S=2048")
    wl = synth.WORKLOADS["s8192"]
    S, c, topk, H, D = 2048, 4, 64, 16, 128
    x = synth.make_inputs(wl, parts=("route",), S=S)
    rng = np.random.default_rng(31)
    logits = synth.to_bf16_values(rng.standard_normal((1, S, D)).astype(np.float32))
    NB = S // c
    src = (np.arange(NB)[:, None] * c + np.arange(c)[None, :]).astype(np.int32)[None]
    valid = np.ones_like(src, dtype=bool)
    k_d = to_dev(x["kI"], torch.bfloat16)
    pk, pz = irb.gather_region_payload(k_d, to_dev(logits, torch.bfloat16), to_dev(src), to_dev(valid))
    summ = irb.summarize_region_payload(pk, pz, to_dev(valid))
    rpk, rpz = oracle.gather_region_payload(x["kI"], logits, src, valid)
    _check_summaries(host(summ).astype(np.float64), rpk, rpz, valid)
    q_e4 = irb.round_e4m3(to_dev(x["qI"], torch.bfloat16))
    qe_h = oracle.round_to_e4m3(x["qI"])
    np.testing.assert_array_equal(host(q_e4), qe_h)
    # the oracle's E4M3 queries and summaries (exact in bf16 and FP32) feed both
    # sides of the scoring; only exact products and FP32 sums separate them
    kc_h = oracle.summarize_region_payload(rpk, rpz, valid)
    scale = 1.0 / math.sqrt(D)
    sc = irb.indexer_score_tile(to_dev(qe_h, torch.bfloat16), to_dev(x["w"]), to_dev(kc_h.astype(np.float32)), c, 0, S,
                                0, NB, scale)
    ref = oracle.indexer_scores(qe_h, x["w"], kc_h, c, scale)
    fin = np.isfinite(ref)
    M = score_bound(qe_h, x["w"], kc_h, scale)
    assert np.array_equal(np.isneginf(host(sc)), ~fin)
    assert np.all(np.abs(host(sc)[fin] - ref[fin]) <= SCORE_ERR * M[fin] + 1e-30)
    ids, cnt = irb.select_regions_csa(sc, c, topk, S)
    rids, rcnt = oracle.select_regions_csa(ref, c, topk)
    got_ids = host(ids)
    np.testing.assert_array_equal(host(cnt), rcnt)
    same = np.all(got_ids == rids, axis=-1)[0]
    # rows that differ must be near ties among the historical scores (k-th and
    # (k+1)-th within 1e-4 relative, as for the block selection)
    ties = np.zeros(S, dtype=bool)
    for t in range(S):
        h = t // c
        if h > topk:
            v = np.sort(ref[0, t, :h])[::-1]
            ties[t] = v[topk - 1] == v[topk] or abs(v[topk - 1] - v[topk]) <= 1e-4 * max(abs(v[topk - 1]), abs(v[topk]))
    bad = ~same & ~ties
    print(f"  csa selection: {int((~same).sum())} rows differ, near-tie rows {int(ties.sum())}")
    assert not bad.any(), np.argwhere(bad)[:5]
