"""Pins of the oracle's per-KV-group routes: grouped scores against a pure-Python
brute force, grouped attention against torch's dense attention with per-head
masks and its autograd, and the reductions to the shared-route functions."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _brute_scores(qI, w, kc, c, scale, docs_of_row):
    """Literal loops over (group, row, query, block, head): no matrix products."""
    B, S, R, H, D = qI.shape
    NB = kc.shape[1]
    out = np.full((R, B, S, NB), -np.inf)
    for b in range(B):
        base = 0
        info = {}
        for (s0, s1) in docs_of_row[b]:
            for t in range(s0, s1):
                info[t] = (base, (t - s0 + 1) // c)
            base += (s1 - s0) // c
        for g in range(R):
            for t in range(S):
                if t not in info:
                    continue
                b0, nb = info[t]
                for j in range(b0, b0 + nb):
                    acc = 0.0
                    for h in range(H):
                        dot = 0.0
                        for d in range(D):
                            dot += float(qI[b, t, g, h, d]) * float(kc[b, j, d])
                        acc += float(w[b, t, g, h]) * max(0.0, dot)
                    out[g, b, t, j] = scale * acc
    return out


def test_grouped_scores_brute_force_packed():
    rng = np.random.default_rng(71)
    B, S, R, H, D, c = 1, 19, 3, 2, 5, 3
    cu = np.array([0, 7, 16], dtype=np.int32)          # two documents, three padding tokens
    qI = rng.standard_normal((B, S, R, H, D))
    w = rng.standard_normal((B, S, R, H))
    kc = rng.standard_normal((B, S // c, D))
    got = oracle.indexer_scores_grouped(qI, w, kc, c, scale=0.37, cu_seqlens=cu)
    want = _brute_scores(qI, w, kc, c, 0.37, [[(0, 7), (7, 16)]])
    assert got.shape == (R, B, S, S // c)
    np.testing.assert_array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)
    # the groups differ (a swapped group / batch axis or a shared group would not)
    assert not np.allclose(got[0][fin[0]], got[1][fin[1]])


def test_grouped_scores_brute_force_batch_rows():
    rng = np.random.default_rng(72)
    B, S, R, H, D, c = 2, 11, 2, 3, 4, 2
    qI = rng.standard_normal((B, S, R, H, D))
    w = rng.standard_normal((B, S, R, H))
    kc = rng.standard_normal((B, S // c, D))
    got = oracle.indexer_scores_grouped(qI, w, kc, c)
    want = _brute_scores(qI, w, kc, c, 1.0 / math.sqrt(D), [[(0, S)], [(0, S)]])
    fin = np.isfinite(want)
    np.testing.assert_array_equal(np.isfinite(got), fin)
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)


def test_one_group_is_the_shared_score():
    rng = np.random.default_rng(73)
    B, S, H, D, c = 1, 24, 4, 8, 4
    qI = rng.standard_normal((B, S, 1, H, D))
    w = rng.standard_normal((B, S, 1, H))
    kc = rng.standard_normal((B, S // c, D))
    got = oracle.indexer_scores_grouped(qI, w, kc, c)
    want = oracle.indexer_scores(qI[:, :, 0], w[:, :, 0], kc, c)
    np.testing.assert_array_equal(got[0], want)


def _group_routes(rng, R, B, S, width, empty=()):
    routes, lens = [], []
    for g in range(R):
        ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.3)
        r, n, _ = oracle.compact_routes(ids, S)
        for (gg, b, t) in empty:
            if gg == g:
                r[b, t] = -1
                n[b, t] = 0
        routes.append(r)
        lens.append(n)
    return np.stack(routes), np.stack(lens)


def _head_masks(routes, lens, Hq, Hkv, S_k):
    """Dense boolean key mask [B, Hq, S_q, S_k]: head h reads the route of KV group h // (Hq/Hkv)."""
    R, B, S_q, _ = routes.shape
    G = Hq // Hkv
    m = np.zeros((B, Hq, S_q, S_k), dtype=bool)
    for h in range(Hq):
        g = h // G if R > 1 else 0
        for b in range(B):
            for t in range(S_q):
                m[b, h, t, routes[g, b, t, :lens[g, b, t]]] = True
    return m


def _sdpa_heads(q, k, v, mask, scale):
    """torch dense attention with per-head masks; empty rows get a dummy key and are zeroed."""
    G = q.shape[2] // k.shape[2]
    mt = torch.as_tensor(mask)
    empty = ~mt.any(-1, keepdim=True)
    mt = mt | (empty & (torch.arange(mask.shape[-1]) == 0))
    out = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), k.repeat_interleave(G, 2).permute(0, 2, 1, 3),
                                         v.repeat_interleave(G, 2).permute(0, 2, 1, 3), attn_mask=mt, scale=scale)
    keep = (~empty).permute(0, 2, 1, 3)                    # [B, S_q, Hq, 1]
    out = out.permute(0, 2, 1, 3)
    return torch.where(keep, out, torch.zeros_like(out))


@pytest.mark.parametrize("Hq,Hkv,B", [(4, 2, 1), (6, 3, 2), (8, 4, 1)])
def test_grouped_forward_equals_dense_per_head_masks(Hq, Hkv, B):
    rng = np.random.default_rng(74 + Hq)
    S, D, Dv = 21, 8, 6
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    routes, lens = _group_routes(rng, Hkv, B, S, 6, empty=[(1, 0, 5)])
    o, lse = oracle.attention_fwd_grouped(q, k, v, routes, 0.53)
    mask = _head_masks(routes, lens, Hq, Hkv, S)
    want = _sdpa_heads(*(torch.as_tensor(x) for x in (q, k, v)), mask, 0.53).numpy()
    np.testing.assert_allclose(o, want, rtol=1e-10, atol=1e-12)
    # lse = logsumexp over the head's own route; -inf for an empty route
    x = 0.53 * np.einsum("bthd,bshd->bhts", q, np.repeat(k, Hq // Hkv, axis=2))
    x = np.where(mask, x, -np.inf)
    with np.errstate(divide="ignore"):
        m = x.max(-1)
        want_lse = np.where(np.isfinite(m), m + np.log(np.exp(x - np.where(np.isfinite(m), m, 0)[..., None]).sum(-1)), -np.inf)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)
    assert lse[0, (Hq // Hkv) * 1, 5] == -np.inf and lse[0, 0, 5] > -np.inf


def test_grouped_backward_equals_autograd_of_dense_form():
    rng = np.random.default_rng(81)
    B, S, Hq, Hkv, D, Dv = 1, 17, 6, 3, 5, 4
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    dO = rng.standard_normal((B, S, Hq, Dv))
    routes, lens = _group_routes(rng, Hkv, B, S, 5, empty=[(2, 0, 3)])
    dq, dk, dv = oracle.attention_bwd_grouped(q, k, v, routes, dO, 0.7)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = _sdpa_heads(qt, kt, vt, _head_masks(routes, lens, Hq, Hkv, S), 0.7)
    (out * torch.as_tensor(dO)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_identical_group_routes_reduce_to_shared_routes():
    rng = np.random.default_rng(82)
    B, S, Hq, Hkv, D = 1, 15, 4, 2, 6
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, D))
    dO = rng.standard_normal((B, S, Hq, D))
    routes, lens = _group_routes(rng, 1, B, S, 6)
    both = np.concatenate([routes, routes])
    o1, l1 = oracle.attention_fwd_grouped(q, k, v, both)
    o0, l0 = oracle.attention_fwd(q, k, v, routes[0])
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l0, rtol=1e-13, atol=1e-14)
    g1 = oracle.attention_bwd_grouped(q, k, v, both, dO)
    g0 = oracle.attention_bwd(q, k, v, routes[0], dO)
    for a, b in zip(g1, g0):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_route_group_count_is_checked():
    q = np.zeros((1, 4, 4, 2)); k = np.zeros((1, 4, 2, 2))
    with pytest.raises(ValueError):
        oracle.attention_fwd_grouped(q, k, k, np.zeros((3, 1, 4, 2), dtype=np.int32))
