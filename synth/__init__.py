"""Seeded synthetic inputs for learned-indexer routed sparse attention.

This module only draws random tensors, in the shapes, dtypes and value
distributions of the five workloads below, and hands them out as plain NumPy
arrays.  It computes nothing the method computes: it holds no compression,
scoring, selection, routing or attention arithmetic.  Both the FP64 oracle
and the GPU path consume exactly the arrays produced here.

Conventions
-----------
* Every tensor of a workload is drawn from its own child of
  ``SeedSequence(base_seed)`` (``PCG64``), children spawned in the fixed order
  of ``TENSOR_ORDER``, so drawing a subset never shifts the others.
* "bf16" tensors are returned as float32 arrays whose values are exactly
  representable in bfloat16 (round-to-nearest-even applied here); the GPU
  side converts them to bfloat16 without further rounding and the oracle
  widens them to float64 exactly.
* Rotary tables are model inputs (the indexer receives them ready-made), laid
  out per token as ``cat(cos, sin)`` over ``D_rope/2`` frequencies, at each
  token's document-relative position, base theta = 10000.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

TENSOR_ORDER = ("layout", "kI", "qI", "w", "gamma", "q", "k", "v", "dO", "idx", "draws")


def _children(base_seed: int) -> dict:
    kids = np.random.SeedSequence(base_seed).spawn(len(TENSOR_ORDER))
    return {name: np.random.Generator(np.random.PCG64(k)) for name, k in zip(TENSOR_ORDER, kids)}


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    _round_bf16_inplace(x)
    return x


def _round_bf16_inplace(x: np.ndarray) -> None:
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    bits += np.uint32(0x7FFF)
    bits += lsb
    bits &= np.uint32(0xFFFF0000)


_CHUNK = 1 << 21            # elements per independently seeded piece of a tensor
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _normal(rng, shape, dtype: str, rms_rows: bool = False, scale: float = 1.0) -> np.ndarray:
    """N(0,1) float32 tensor drawn in row-aligned pieces, each from its own PCG64 seeded by ``rng``.

    The pieces are filled by a thread pool (NumPy's generators and ufuncs run
    without the GIL), so drawing a 10^9-element tensor takes seconds.  The
    values depend only on ``rng``'s state and ``shape``.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    n = out.size
    if n == 0:
        return out
    row = shape[-1] if shape else 1
    flat = out.reshape(-1, row)
    rows_per = max(1, _CHUNK // row)
    starts = list(range(0, flat.shape[0], rows_per))
    seeds = rng.integers(0, 2 ** 63, size=len(starts), dtype=np.int64)

    def fill(i):
        piece = flat[starts[i]:starts[i] + rows_per]
        np.random.Generator(np.random.PCG64(int(seeds[i]))).standard_normal(piece.shape, dtype=np.float32, out=piece)
        if rms_rows:
            # per-head RMS normalisation of the last axis: x / sqrt(mean(x^2))
            ms = np.mean(np.square(piece, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
            piece /= np.sqrt(ms)
        if scale != 1.0:
            piece *= np.float32(scale)
        if dtype == "bf16":
            _round_bf16_inplace(piece)

    if len(starts) == 1:
        fill(0)
    else:
        with concurrent.futures.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def rope_table(doc_pos: np.ndarray, d_rope: int, theta: float = 10000.0) -> np.ndarray:
    """Rotary input table [..., d_rope] = cat(cos, sin) at the given positions (float32)."""
    half = d_rope // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d_rope)
    ang = doc_pos.astype(np.float64)[..., None] * inv
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def doc_positions(B: int, S: int, cu_seqlens: Optional[np.ndarray], row_lens: Optional[np.ndarray]) -> np.ndarray:
    """Document-relative position of every physical token (0 on padding)."""
    pos = np.zeros((B, S), dtype=np.int64)
    if cu_seqlens is not None:
        for d in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[d]), int(cu_seqlens[d + 1])
            pos[0, a:e] = np.arange(e - a)
    else:
        for b in range(B):
            n = S if row_lens is None else int(row_lens[b])
            pos[b, :n] = np.arange(n)
    return pos


def varlen_documents(rng, total: int, min_len: int = 256, max_len: int = 16384, max_pad: int = 511):
    """Packed layout: log-uniform document lengths filling ``total - pad`` tokens.

    ``pad`` ~ U{0..max_pad}; the last document is truncated to fit.  Returns
    ``(cu_seqlens int32 [docs+1], pad)``.
    """
    pad = int(rng.integers(0, max_pad + 1))
    budget = total - pad
    lens = []
    filled = 0
    while filled < budget:
        n = int(math.floor(math.exp(rng.uniform(math.log(min_len), math.log(max_len)))))
        n = min(n, budget - filled)
        lens.append(n)
        filled += n
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return cu, pad


def latent_indices(rng, T: int, width: int) -> np.ndarray:
    """Causal random index lists [T, 1, width]: a random valid prefix, -1 after.

    For each query t: n ~ U{1..width}, m = min(n, t+1) distinct IDs drawn
    uniformly from [0, t], placed in random order in the first m slots.
    """
    out = np.full((T, 1, width), -1, dtype=np.int32)
    n = rng.integers(1, width + 1, size=T)
    for t in range(T):
        m = int(min(n[t], t + 1))
        out[t, 0, :m] = rng.choice(t + 1, size=m, replace=False)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    S: int
    dtype: str              # activation dtype of q/k/v and indexer states: "f32" or "bf16"
    # route pipeline (None for the latent workload, whose routes are given)
    H_idx: int = 0
    D_idx: int = 0
    c: int = 0
    topk: int = 0
    window: int = 0
    packed: bool = False
    w_std: float = 1.0
    # attention
    Hq: int = 0
    Hkv: int = 0
    D: int = 0
    Dv: int = 0
    latent: bool = False
    latent_width: int = 0
    softmax_scale: Optional[float] = None
    rms_inputs: bool = False
    backward: bool = False
    description: str = ""

    @property
    def route_width(self) -> int:
        if self.latent:
            return self.latent_width
        return self.topk * self.c + max(self.window, self.c - 1)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=1000, B=1, S=512, dtype="f32", H_idx=4, D_idx=64, c=4, topk=16, window=0,
        w_std=1.0 / math.sqrt(4), Hq=4, Hkv=1, D=64, Dv=64, backward=True,
        description="B=1 S=512 one causal document, fp32; indexer 4x64, c=4, top-16 blocks; attention 4/1 heads, D=64"),
    "s8192": Workload(
        name="s8192", seed=1001, B=1, S=8192, dtype="bf16", H_idx=16, D_idx=128, c=4, topk=512, window=128,
        w_std=1.0 / 4.0, Hq=32, Hkv=4, D=128, Dv=128, rms_inputs=True, backward=False,
        description="B=1 S=8192 one causal document, bf16; indexer 16x128, c=4, top-512 blocks + 128-token window; GQA 32/4, D=128; forward"),
    "varlen": Workload(
        name="varlen", seed=1002, B=1, S=32768, dtype="bf16", H_idx=16, D_idx=128, c=4, topk=256, window=0,
        packed=True, w_std=1.0 / 4.0, Hq=32, Hkv=4, D=128, Dv=128, rms_inputs=True, backward=True,
        description="packed T=32768, log-uniform documents in [256,16384] + 0-511 padding tail; indexer 16x128, c=4, top-256; GQA 32/4, D=128; fwd+bwd"),
    "latent": Workload(
        name="latent", seed=1003, B=1, S=16384, dtype="bf16", Hq=64, Hkv=1, D=576, Dv=512, latent=True,
        latent_width=2048, softmax_scale=1.0 / 24.0, backward=True,
        description="latent single-KV-head: T=16384, 64 heads, q/k dim 576, value dim 512, causal random index lists width 2048; fwd+bwd"),
    "long": Workload(
        name="long", seed=1004, B=1, S=131072, dtype="bf16", H_idx=32, D_idx=128, c=8, topk=256, window=512,
        w_std=1.0 / math.sqrt(32), Hq=64, Hkv=8, D=128, Dv=128, rms_inputs=True, backward=True,
        description="B=1 S=131072 one causal document; indexer 32x128, c=8, top-256 + 512-token window; GQA 64/8, D=128; fwd+bwd"),
}


def make_layout(wl: Workload, rngs=None):
    """Return (cu_seqlens or None, row_lens or None) for a workload."""
    if wl.packed:
        rngs = rngs or _children(wl.seed)
        cu, _pad = varlen_documents(rngs["layout"], wl.S)
        return cu, None
    return None, None


def make_inputs(wl: Workload, parts=("route", "attn"), S: Optional[int] = None,
                cu_seqlens: Optional[np.ndarray] = None, row_lens: Optional[np.ndarray] = None,
                B: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Draw the inputs of a workload.

    ``parts`` selects "route" (indexer states, weights, rotary table), "attn"
    (q, k, v), "bwd" (dO), "draws" (uniform numbers, one per row and
    selection slot) and, for the latent workload, "idx".  ``S``, ``B``,
    ``cu_seqlens``, ``row_lens`` and ``seed`` override the workload's own
    values so that tests can draw the same recipe at smaller sizes.
    """
    B = wl.B if B is None else B
    S = wl.S if S is None else S
    rngs = _children(wl.seed if seed is None else seed)
    out: dict = {"B": B, "S": S, "workload": wl.name}
    if cu_seqlens is None and row_lens is None and wl.packed and S == wl.S and B == 1:
        cu_seqlens, _ = make_layout(wl, rngs)
    out["cu_seqlens"] = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32)
    out["row_lens"] = None if row_lens is None else np.asarray(row_lens, dtype=np.int32)
    dt = wl.dtype
    if "route" in parts and not wl.latent:
        out["kI"] = _normal(rngs["kI"], (B, S, wl.D_idx), dt)
        out["qI"] = _normal(rngs["qI"], (B, S, wl.H_idx, wl.D_idx), dt, rms_rows=wl.rms_inputs)
        out["w"] = _normal(rngs["w"], (B, S, wl.H_idx), "f32", scale=wl.w_std)
        out["gamma"] = np.ones(wl.D_idx, dtype=np.float32)
        pos = doc_positions(B, S, out["cu_seqlens"], out["row_lens"])
        out["freqs"] = rope_table(pos, wl.D_idx)
    if "attn" in parts:
        if wl.latent:
            out["q"] = _normal(rngs["q"], (S, wl.Hq, wl.D), dt)
            out["kv"] = _normal(rngs["k"], (S, 1, wl.D), dt)
        else:
            out["q"] = _normal(rngs["q"], (B, S, wl.Hq, wl.D), dt, rms_rows=wl.rms_inputs)
            out["k"] = _normal(rngs["k"], (B, S, wl.Hkv, wl.D), dt, rms_rows=wl.rms_inputs)
            out["v"] = _normal(rngs["v"], (B, S, wl.Hkv, wl.Dv), dt, rms_rows=wl.rms_inputs)
    if "bwd" in parts:
        if wl.latent:
            out["dO"] = _normal(rngs["dO"], (S, wl.Hq, wl.Dv), dt)
        else:
            out["dO"] = _normal(rngs["dO"], (B, S, wl.Hq, wl.Dv), dt)
    if "idx" in parts and wl.latent:
        out["idx"] = latent_indices(rngs["idx"], S, wl.latent_width)
    if "draws" in parts and not wl.latent:
        # uniform [0, 1) per (row, selection slot): a stand-in for block choices when a
        # test needs routes at full size without scoring every block
        out["draws"] = rngs["draws"].random((B, S, wl.topk), dtype=np.float32)
    return out


def random_routes(rng, B: int, S: int, width: int, causal: bool = True, frac_invalid: float = 0.1,
                  duplicates: bool = True) -> np.ndarray:
    """Unsorted signed ID lists [B, S, width] for compaction tests.

    IDs are drawn from [0, t] when ``causal`` (else from [0, S)), a fraction
    set to -1 or to out-of-range values, optionally with repeats.
    """
    out = np.empty((B, S, width), dtype=np.int32)
    for b in range(B):
        for t in range(S):
            hi = t + 1 if causal else S
            ids = rng.integers(0, hi, size=width)
            if not duplicates:
                m = min(width, hi)
                ids = np.full(width, -1, dtype=np.int64)
                ids[:m] = rng.choice(hi, size=m, replace=False)
            bad = rng.random(width) < frac_invalid
            ids = np.where(bad, rng.choice(np.array([-1, -7, S, S + 5]), size=width), ids)
            out[b, t] = ids
    return out
