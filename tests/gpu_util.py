"""Shared helpers of the GPU parity tests (test infrastructure only)."""
import math

import numpy as np
import torch

import indexer_routed_block_amd as irb

DEV = "cuda"


def to_dev(x, dtype=None):
    """Upload a NumPy array, converting on the device (bf16 inputs are exactly representable)."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if dtype is not None:
        t = t.to(dtype)
    return t


def act_dtype(wl_dtype):
    return torch.bfloat16 if wl_dtype == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x|: 2^(floor(log2|x|) - 8) (8 significand bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def bf16_tolerance(want):
    """Per-element bound on a bf16 attention output / gradient against the FP64 value.

    2e-2 absolute (the stated max-abs bound) wherever |ref| < 4; from |ref| >= 4
    on, 2e-2 plus one bf16 storage half-ulp of the value, the error that
    storing the FP32-accumulated result in bf16 can add on its own (a value in
    [16, 32) cannot be stored closer than 0.0625).  Keys shared by many
    queries have gradients of that size; unit-scale values get no relaxation.
    """
    a = np.abs(np.asarray(want, dtype=np.float64))
    return np.where(a < 4.0, 2e-2, 2e-2 + bf16_half_ulp(a))


def attn_tol_check(got, want, dtype, what):
    """Attention outputs / gradients against the FP64 oracle.

    bf16: mean-abs <= 5e-3, and per element |err| <= bf16_tolerance(ref).
    The worst error among |ref| < 4 elements (where the bound is the plain
    2e-2) and the overall max-abs are printed.  fp32 inputs: max-abs <= 1e-4.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    scale = float(np.abs(want).max(initial=0.0))
    small = np.abs(want) < 4.0
    mx_small = float(err[small].max(initial=0.0))
    if dtype == torch.bfloat16:
        over = err - bf16_tolerance(want)
        worst = float(over.max(initial=-1.0))
        ok = worst <= 0.0 and mean <= 5e-3
    else:
        worst = mx - 1e-4
        ok = mx <= 1e-4
    print(f"  {what}: max-abs {mx:.3e} (|ref|<4: {mx_small:.3e}) mean-abs {mean:.3e} max|ref| {scale:.3f}")
    if not ok and err.size:
        bad = np.argwhere(err > (bf16_tolerance(want) if dtype == torch.bfloat16 else 1e-4))
        print(f"  {what}: {len(bad)} elements beyond the bound; first {bad[:8].tolist()}; worst at "
              f"{np.unravel_index(int(np.argmax(err)), err.shape)}")
    assert ok, (f"{what}: max-abs {mx:.3e}, |ref|<4 max-abs {mx_small:.3e}, worst excess over the bound "
                f"{worst:.3e}, mean-abs {mean:.3e} (max |ref| {scale:.3f})")
    return mx, mean


# FP32 scoring error bound, relative to the magnitude M = scale sum_h |w| sum_d |q k|:
# keys carried as bf16 high + low parts (2^-16 of each key), FP32 accumulation
# over D = 128 products (128 * 2^-24) and over the heads: < 3e-5 M.
SCORE_ERR = 3e-5


def check_selection(wl, x, topk, got, ref, kc, grouped, extra=None):
    """GPU selections and routes against the oracle's, every row.

    ``got`` / ``ref``: dicts of NumPy arrays sel, cnt, routes, lens with a
    leading route-group axis ([R, B, S, ...]; shared routes R = 1); ``ref``
    also holds the oracle's near-tie rows ``ties`` [R, B, S].

    Counts always agree.  Rows whose selection equals the oracle's are
    compared bit for bit (selection, routes, lengths).  A row that differs
    must still be a correct top-k under FP32 scoring: some perturbation of
    each score by at most SCORE_ERR * M makes the GPU's set the top k, and its
    routes must be the oracle's expansion of the GPU's own selection.  With
    shared routes a differing row must moreover be one of the oracle's near
    ties (k-th and (k+1)-th scores within 1e-4 relative); per-group scores of
    a few signed-weight heads cancel far below that relative precision, so
    there every row takes the validity check.  ``extra(b, t)``, when given,
    widens the perturbation by a further bound per block of row (b, t) (a
    known ambiguity of the scored inputs themselves); a differing row then
    takes the validity check whether or not it is a near tie.  Returns
    (near-tie rows, differing rows).
    """
    import oracle

    np.testing.assert_array_equal(got["cnt"], ref["cnt"])
    assert got["sel"].shape == ref["sel"].shape and got["routes"].shape == ref["routes"].shape
    same = np.all(got["sel"] == ref["sel"], axis=-1)
    np.testing.assert_array_equal(got["routes"][same], ref["routes"][same])
    np.testing.assert_array_equal(got["lens"][same], ref["lens"][same])
    ties = ref["ties"]
    if not grouped and extra is None:
        bad = ~same & ~ties
        assert not bad.any(), f"{int(bad.sum())} non-tie rows differ, e.g. {np.argwhere(bad)[:3].tolist()}"
    diff = np.argwhere(~same)
    print(f"  selection: near-tie rows {int(ties.sum())}, rows differing from the oracle {len(diff)} of {same.size}")
    scale = 1.0 / math.sqrt(wl.D_idx)
    cu, rl = x["cu_seqlens"], x["row_lens"]
    B, S = got["sel"].shape[1], got["sel"].shape[2]
    docs = oracle.documents(B, S, cu, rl)
    valid, start, base, nb = oracle.token_info(docs, S, wl.c)
    for g, b, t in diff:
        if grouped:
            s = oracle.indexer_scores_grouped(x["qI"], x["w"], kc, wl.c, scale, cu, rl, q0=t, q1=t + 1)[g, b, 0]
            M = score_bound(x["qI"][b:b + 1, t:t + 1, g], x["w"][b:b + 1, t:t + 1, g], kc[b:b + 1], scale)[0, 0]
        else:
            s = oracle.indexer_scores(x["qI"], x["w"], kc, wl.c, scale, cu, rl, q0=t, q1=t + 1)[b, 0]
            M = score_bound(x["qI"][b:b + 1, t:t + 1], x["w"][b:b + 1, t:t + 1], kc[b:b + 1], scale)[0, 0]
        lo, n = int(base[b, t]), int(nb[b, t])
        k = int(got["cnt"][g, b, t])
        chosen = got["sel"][g, b, t, :k] - lo
        assert k == min(topk, n) and len(set(chosen.tolist())) == k and np.all((chosen >= 0) & (chosen < n))
        assert np.all(got["sel"][g, b, t, k:] == -1)
        inside = np.zeros(n, dtype=bool)
        inside[chosen] = True
        vs, vm = s[lo:lo + n], SCORE_ERR * M[lo:lo + n]
        if extra is not None:
            vm = vm + extra(b, t)[lo:lo + n]
        if k < n:
            low = np.min(vs[inside] + vm[inside])
            high = np.max(vs[~inside] - vm[~inside])
            assert low >= high, f"group {g} row {b},{t}: not a top-{k} within the FP32 bound ({low:.3e} < {high:.3e})"
        sel1 = got["sel"][g, b:b + 1].copy()
        cnt1 = got["cnt"][g, b:b + 1].copy()
        rr, ll = oracle.expand_routes(sel1, cnt1, wl.c, wl.window, topk, cu,
                                      None if rl is None else rl[b:b + 1], rows=[(0, int(t))])
        np.testing.assert_array_equal(got["routes"][g, b, t], rr[0, t])
        assert got["lens"][g, b, t] == ll[0, t]
    return int(ties.sum()), len(diff)


def score_bound(qI, w, kc, scale):
    """M[b, t, j] = scale * sum_h |w[t,h]| * sum_d |q[t,h,d] k[j,d]|.

    The "1e-3 relative" score tolerance is taken against this magnitude: it
    bounds the cancellation inside each dot product as well as across the
    signed head weights, so it is the scale FP32-class rounding error lives
    on.  (relu(q.k) alone is not: a dot product that cancels to ~0 still
    carries rounding error of order sum_d |q_d k_d| * 2^-17.)
    """
    dots = np.abs(qI.astype(np.float64)) @ np.abs(np.asarray(kc, dtype=np.float64)).swapaxes(-1, -2)[:, None]
    return scale * (np.abs(w.astype(np.float64))[..., None, :] @ dots)[..., 0, :]


def rne_bf16(y):
    """Round float64 values to the nearest bf16 (8 significant bits), ties to even."""
    f, e = np.frexp(y)                      # y = f 2^e, |f| in [0.5, 1)
    return np.ldexp(np.rint(f * 256.0), e - 8)


def prep_term_bound(q, gamma, freqs, d_rope):
    """FP32 error bound E per element of the prepared index queries: 2^-20 times
    the summed magnitudes of the terms combined (|u_i cos| + |u_p sin| for a
    rotated dimension, |u_i| otherwise; u the normalised row)."""
    import oracle

    u = np.abs(oracle.prepare_index_queries(q, gamma, freqs, 1e-5, d_rope=0))
    mag = u.copy()
    h = d_rope // 2
    if h:
        cos = np.abs(freqs[..., :h])[:, :, None, :]
        sin = np.abs(freqs[..., h:2 * h])[:, :, None, :]
        mag[..., :h] = u[..., :h] * cos + u[..., h:2 * h] * sin
        mag[..., h:2 * h] = u[..., h:2 * h] * cos + u[..., :h] * sin
    return 2.0 ** -20 * (mag + 1e-30)
