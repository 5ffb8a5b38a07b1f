"""GPU parity of irb_prepare_index_queries (index-query RMSNorm + RoPE at the
query's own token) against the FP64 oracle.

bf16 outputs: the kernel rounds its FP32 result once to bf16 (round to nearest
even), so each element must be the bf16 rounding of a value within the FP32
arithmetic's error of the oracle's FP64 value y: RNE(y - E) <= got <= RNE(y + E)
with E = 2^-20 * (the magnitudes of the terms combined: |u_i cos| + |u_p sin|
for a rotated dimension, |u_i| otherwise, u the normalised row).  Elements that
differ from RNE(y) are counted and printed (they are rounding-boundary cases
and RoPE cancellations).  FP32 outputs: within 1e-5 of the oracle, relative to
max(1, |value|)."""
import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import banner, host, prep_term_bound as _term_bound, rne_bf16 as _rne_bf16, to_dev

pytestmark = pytest.mark.gpu


def _check_bf16(got, ref, bound):
    lo, hi = _rne_bf16(ref - bound), _rne_bf16(ref + bound)
    ok = (got >= lo) & (got <= hi)
    bad = np.argwhere(~ok)
    assert bad.size == 0, (f"{bad.shape[0]} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]} "
                           f"ref {ref[tuple(bad[0])]} bound {bound[tuple(bad[0])]}")
    return int(np.sum(got != _rne_bf16(ref)))


def _case(rng, B, S, H, D, d_rope, cu=None):
    q = rng.standard_normal((B, S, H, D)) * rng.uniform(0.1, 5.0, (B, S, H, 1))
    gamma = rng.uniform(0.5, 1.5, D).astype(np.float32)
    pos = synth.doc_positions(B, S, cu, None)
    freqs = synth.rope_table(pos, d_rope) if d_rope else np.zeros((B, S, 0), np.float32)
    return q.astype(np.float32), gamma, freqs


@pytest.mark.parametrize("D,d_rope,H,S", [(128, 128, 16, 333), (128, 64, 4, 300), (64, 64, 3, 129), (32, 0, 2, 77),
                                          (256, 6, 2, 50), (512, 512, 1, 40), (64, 16, 8, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prepare_index_queries_matches_oracle(D, d_rope, H, S, dtype):
    banner(f"prepare queries D={D} D_rope={d_rope} H={H} S={S} {dtype}")
    rng = np.random.default_rng(D + d_rope + H + S)
    cu = np.array([0, S // 3, S], dtype=np.int32) if S > 3 else None
    q, gamma, freqs = _case(rng, 1, S, H, D, d_rope, cu)
    if dtype == "bf16":
        q = synth.to_bf16_values(q)          # exactly representable: both sides see the same inputs
        qd = to_dev(q, torch.bfloat16)
    else:
        qd = to_dev(q)
    g = to_dev(gamma)
    fr = to_dev(freqs) if d_rope else None
    out = irb.prepare_index_queries(qd, g, fr, 1e-5)
    ref = oracle.prepare_index_queries(q.astype(np.float64), gamma, freqs, 1e-5, d_rope=d_rope)
    got = out.float().cpu().numpy().astype(np.float64)
    if dtype == "bf16":
        off = _check_bf16(got, ref, _term_bound(q.astype(np.float64), gamma, freqs, d_rope))
        print(f"elements off RNE(oracle) within the FP32 error: {off} of {ref.size}")
    else:
        assert np.all(np.abs(got - ref) <= 1e-5 * np.maximum(1.0, np.abs(ref)))
    # in place: the output may alias the input
    qi = qd.clone()
    irb.prepare_index_queries(qi, g, fr, 1e-5, out=qi)
    assert torch.equal(qi, out)


def test_prepare_index_queries_full_size_long_recipe():
    """The 131072-token, 32-head, 128-dim index queries of the long-context
    workload, with its rotary table; sampled token rows against the oracle."""
    wl = synth.WORKLOADS["long"]
    S, H, D = wl.S, wl.H_idx, wl.D_idx
    banner(f"prepare queries full size S={S} H={H} D={D}")
    rng = np.random.default_rng(1234)
    qd = torch.randn((1, S, H, D), generator=torch.Generator().manual_seed(5), dtype=torch.float32).to("cuda").to(torch.bfloat16)
    gamma = rng.uniform(0.5, 1.5, D).astype(np.float32)
    freqs = synth.rope_table(np.arange(S)[None], D)
    out = irb.prepare_index_queries(qd, to_dev(gamma), to_dev(freqs), 1e-5)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(S - 8, S), rng.integers(0, S, 48)]))
    qs = qd[:, rows].float().cpu().numpy().astype(np.float64)
    ref = oracle.prepare_index_queries(qs, gamma, freqs[:, rows], 1e-5)
    got = out[:, rows].float().cpu().numpy().astype(np.float64)
    off = _check_bf16(got, ref, _term_bound(qs, gamma, freqs[:, rows], D))
    print(f"elements off RNE(oracle) within the FP32 error: {off} of {ref.size}")
