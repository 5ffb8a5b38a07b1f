"""Pins of the oracle's sparse attention against torch's dense attention, autograd and finite differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _dense_mask(routes, lens, S_k):
    B, S_q, _ = routes.shape
    m = np.zeros((B, S_q, S_k), dtype=bool)
    for b in range(B):
        for t in range(S_q):
            m[b, t, routes[b, t, :lens[b, t]]] = True
    return m


def _sdpa(q, k, v, mask, scale):
    """torch FP64 dense attention with a boolean key mask, GQA by repeating K/V heads."""
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    qt = torch.as_tensor(q).permute(0, 2, 1, 3)
    kt = torch.as_tensor(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.as_tensor(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    mt = torch.as_tensor(mask)[:, None]
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return out.permute(0, 2, 1, 3)


def _routes(rng, B, S, width, extra_empty=()):
    ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.3)
    routes, lens, _ = oracle.compact_routes(ids, S)
    for (b, t) in extra_empty:
        routes[b, t] = -1
        lens[b, t] = 0
    return routes, lens


@pytest.mark.parametrize("Hq,Hkv,D,Dv", [(4, 1, 16, 16), (6, 2, 8, 12), (8, 8, 4, 4)])
def test_forward_equals_dense_masked_sdpa(Hq, Hkv, D, Dv):
    rng = np.random.default_rng(31)
    B, S = 2, 29
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    routes, lens = _routes(rng, B, S, 9, extra_empty=[(1, 3)])
    scale = 0.37
    o, lse = oracle.attention_fwd(q, k, v, routes, scale)
    mask = _dense_mask(routes, lens, S)
    ref = _sdpa(q, k, v, mask, scale).numpy()
    nonempty = lens > 0
    np.testing.assert_allclose(o[nonempty], ref[nonempty], rtol=1e-10, atol=1e-12)
    assert np.all(o[~nonempty] == 0) and np.all(np.isneginf(lse.transpose(0, 2, 1)[~nonempty]))
    # softmax rows sum to one: sum_k exp(x_k - lse) == 1
    for b in range(B):
        for t in range(S):
            if not lens[b, t]:
                continue
            ids = routes[b, t, :lens[b, t]]
            for h in range(Hq):
                x = scale * k[b, ids, h // (Hq // Hkv)] @ q[b, t, h]
                assert abs(np.exp(x - lse[b, h, t]).sum() - 1.0) < 1e-12


def test_full_prefix_routes_equal_causal_attention():
    rng = np.random.default_rng(32)
    B, S, Hq, Hkv, D = 1, 40, 4, 2, 8
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, D))
    routes = np.full((B, S, S), -1, dtype=np.int32)
    for t in range(S):
        routes[0, t, :t + 1] = np.arange(t + 1)
    o, _ = oracle.attention_fwd(q, k, v, routes)
    G = Hq // Hkv
    ref = F.scaled_dot_product_attention(
        torch.as_tensor(q).permute(0, 2, 1, 3),
        torch.as_tensor(k).repeat_interleave(G, 2).permute(0, 2, 1, 3),
        torch.as_tensor(v).repeat_interleave(G, 2).permute(0, 2, 1, 3), is_causal=True).permute(0, 2, 1, 3)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_window_only_routes_equal_sliding_window_attention():
    # topk = 0 blocks, window W: the route pipeline gives [t-W+1, t]
    rng = np.random.default_rng(33)
    S, c, W = 37, 4, 5
    sel = np.full((1, S, 0), -1, dtype=np.int32)
    cnt = np.zeros((1, S), dtype=np.int32)
    routes, lens = oracle.expand_routes(sel, cnt, c, W, 0)
    q = rng.standard_normal((1, S, 2, 8)); k = rng.standard_normal((1, S, 1, 8)); v = rng.standard_normal((1, S, 1, 8))
    o, _ = oracle.attention_fwd(q, k, v, routes)
    i = np.arange(S)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref = _sdpa(q, k, v, band[None], 1 / np.sqrt(8)).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 1)])
def test_backward_equals_autograd_of_dense_form(Hq, Hkv):
    rng = np.random.default_rng(34)
    B, S, D, Dv = 1, 23, 8, 6
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    dO = rng.standard_normal((B, S, Hq, Dv))
    routes, lens = _routes(rng, B, S, 7, extra_empty=[(0, 4)])
    scale = 0.61
    dq, dk, dv = oracle.attention_bwd(q, k, v, routes, dO, scale)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _dense_mask(routes, lens, S)
    out = _sdpa_t(qt, kt, vt, mask, scale)
    keep = torch.as_tensor(lens > 0)[..., None, None]
    (torch.where(keep, out, torch.zeros_like(out)) * torch.as_tensor(dO)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-9, atol=1e-11)
    # invariants: sum over keys of dV equals the sum of dO over the group's heads and nonempty queries
    G = Hq // Hkv
    for g in range(Hkv):
        want = (dO[0, lens[0] > 0][:, g * G:(g + 1) * G]).sum(axis=(0, 1))
        np.testing.assert_allclose(dv[0, :, g].sum(axis=0), want, rtol=1e-10, atol=1e-10)


def _sdpa_t(q, k, v, mask, scale):
    G = q.shape[2] // k.shape[2]
    mt = torch.as_tensor(mask)[:, None]
    # rows with no key produce NaN in SDPA; give them a dummy key and zero them afterwards
    empty = ~mt.any(-1, keepdim=True)
    mt = mt | (empty & (torch.arange(mask.shape[-1]) == 0))
    out = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), k.repeat_interleave(G, 2).permute(0, 2, 1, 3),
                                         v.repeat_interleave(G, 2).permute(0, 2, 1, 3), attn_mask=mt, scale=scale)
    return out.permute(0, 2, 1, 3)


def test_backward_central_differences():
    rng = np.random.default_rng(35)
    B, S, Hq, Hkv, D, Dv = 1, 9, 2, 1, 3, 2
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    dO = rng.standard_normal((B, S, Hq, Dv))
    routes, lens = _routes(rng, B, S, 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, routes, dO, 0.8)
    f = lambda q_, k_, v_: float(np.sum(oracle.attention_fwd(q_, k_, v_, routes, 0.8)[0] * dO))
    eps = 1e-6
    for arr, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1 = arr.copy(); a1[idx] += eps
            a0 = arr.copy(); a0[idx] -= eps
            args1 = [q, k, v]; args0 = [q, k, v]
            pos = "qkv".index(name)
            args1[pos] = a1; args0[pos] = a0
            num[idx] = (f(*args1) - f(*args0)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-5, atol=1e-7)


def test_latent_merges_key_and_value_gradients():
    rng = np.random.default_rng(36)
    T, H, Dqk, Dv, W = 17, 3, 10, 6, 5
    q = rng.standard_normal((T, H, Dqk)); kv = rng.standard_normal((T, 1, Dqk)); dO = rng.standard_normal((T, H, Dv))
    idx = synth.random_routes(rng, 1, T, W, causal=True, frac_invalid=0.3)[0][:, None, :]
    scale = 0.3
    o, lse = oracle.latent_attention_fwd(q, kv, idx, scale, dv=Dv)
    dq, dkv = oracle.latent_attention_bwd(q, kv, idx, dO, scale, dv=Dv)
    qt = torch.tensor(q, requires_grad=True); kvt = torch.tensor(kv, requires_grad=True)
    routes, lens, _ = oracle.compact_routes(idx[:, 0, :], T)
    mask = _dense_mask(routes[None], lens[None], T)
    out = _sdpa_t(qt[None], kvt[None], kvt[None][..., :Dv], mask, scale)[0]
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-10, atol=1e-12)
    (out * torch.as_tensor(dO)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dkv, kvt.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_duplicates_and_invalid_ids_collapse():
    rng = np.random.default_rng(37)
    q = rng.standard_normal((1, 3, 2, 4)); k = rng.standard_normal((1, 3, 1, 4)); v = rng.standard_normal((1, 3, 1, 4))
    a = np.array([[[0, 1, 2], [0, 1, -1], [2, -1, -1]]], dtype=np.int32)
    b = np.array([[[2, 1, 0, 0, 9, -5], [1, 1, 0, -1, 3, 0], [2, 2, 2, -1, -1, -1]]], dtype=np.int32)
    oa, la = oracle.attention_fwd(q, k, v, a)
    ob, lb = oracle.attention_fwd(q, k, v, b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_restricted_backward_matches_full():
    rng = np.random.default_rng(38)
    B, S, Hq, Hkv, D, Dv = 2, 31, 4, 2, 8, 6
    q = rng.standard_normal((B, S, Hq, D)); k = rng.standard_normal((B, S, Hkv, D)); v = rng.standard_normal((B, S, Hkv, Dv))
    dO = rng.standard_normal((B, S, Hq, Dv))
    routes, lens = _routes(rng, B, S, 9)
    full = oracle.attention_bwd(q, k, v, routes, dO, 0.4)
    rows = [(0, 3), (1, 30), (1, 0)]
    keys = [(0, 0), (0, 17), (1, 29)]
    part = oracle.attention_bwd(q, k, v, routes, dO, 0.4, rows=rows, keys=keys)
    for (b, t) in rows:
        np.testing.assert_array_equal(part[0][b, t], full[0][b, t])
    for (b, kk) in keys:
        np.testing.assert_allclose(part[1][b, kk], full[1][b, kk], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(part[2][b, kk], full[2][b, kk], rtol=1e-12, atol=1e-14)
