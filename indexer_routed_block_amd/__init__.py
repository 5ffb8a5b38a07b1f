"""Python binding of libirb (learned-indexer routed sparse attention, MI355X).

Argument marshalling only: every function below checks what the C library
cannot see through bare pointers (dtype, contiguity, shapes), allocates its
outputs with torch on the tensors' device, and calls the same-named
``irb_*`` entry point on the current HIP stream.  All arithmetic runs in the library's HIP kernels.
There is no fallback: if ``libirb.so`` is missing or no gfx950 device is
current, calls raise ``RuntimeError``.

Status codes map to exceptions as in the latent page's
``cudnn_sparse_attention``: unavailable -> RuntimeError, dtype -> TypeError,
invalid argument -> ValueError, HIP failure -> RuntimeError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libirb.so")

IRB_F32, IRB_BF16 = 0, 1
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class IrbLayout(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("cu_seqlens", _P),
                ("num_docs", ctypes.c_int32), ("row_lens", _P)]


_SIGS = {
    "irb_is_available": ([], _I),
    "irb_last_error": ([], ctypes.c_char_p),
    "irb_version": ([], ctypes.c_char_p),
    "irb_compress_keys": ([_P, _I, _P, _I, _I64, _I64, _I, _P, _F, _P, _I, _P, _P, _P], _I),
    "irb_prepare_index_queries": ([_P, _I, _I64, _I, _I, _P, _F, _P, _I, _P, _P], _I),
    "irb_indexer_score_tile": ([_P, _P, _I, _I, _I, _P, _P, _P, _I, _F, _I, _I, _I, _I, _P, _I64, _P], _I),
    "irb_select_topk_regions": ([_P, _P, _I64, _I, _I, _P, _I, _I, _P, _P, _P], _I),
    "irb_route_topk_fused_workspace_size": ([_I, _I, _I, _I, _I, _I, _I], _SZ),
    "irb_route_topk_fused": ([_P, _P, _I, _I, _I, _P, _P, _P, _I, _F, _I, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "irb_route_topk_fused_raw": ([_P, _P, _I, _I, _I, _P, _F, _P, _I, _P, _P, _P, _I, _F, _I, _I, _I, _P, _P, _P, _SZ,
                                  _P], _I),
    "irb_route_topk_fused_noalloc": ([_P, _P, _I, _I, _I, _P, _P, _P, _I, _F, _I, _I, _I, _P, _P, _P], _I),
    "irb_indexer_score_tile_groups": ([_P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _F, _I, _I, _I, _I, _P, _I64, _P], _I),
    "irb_route_topk_fused_groups_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "irb_route_topk_fused_groups": ([_P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _F, _I, _I, _I, _P, _P, _P, _SZ, _P],
                                    _I),
    "irb_round_e4m3": ([_P, _I, _I64, _P, _P], _I),
    "irb_gather_region_payload": ([_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _P, _P, _P], _I),
    "irb_summarize_region_payload": ([_P, _P, _I, _P, _I, _I, _I, _I, _P, _P], _I),
    "irb_select_regions_csa_workspace_size": ([_I, _I, _I, _I], _SZ),
    "irb_select_regions_csa": ([_P, _P, _I64, _I, _I, _P, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "irb_expand_and_compact_routes": ([_P, _P, _P, _I, _I, _I, _P, _I, _P, _P, _P], _I),
    "irb_compact_routes": ([_P, _I64, _I, _I64, _P, _P, _P, _P], _I),
    "irb_pack_region_bitmap": ([_P, _I64, _I, _I, _P, _P], _I),
    "irb_build_block_lists_workspace_size": ([_I, _I, _I, _I, _I], _SZ),
    "irb_split_full_blocks_workspace_size": ([_I, _I, _I, _I, _I], _SZ),
    "irb_split_full_blocks": ([_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "irb_build_block_lists": ([_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _SZ, _P], _I),
    "irb_sparse_gqa_attention_fwd_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "irb_sparse_gqa_attention_fwd": ([_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P,
                                      _P, _P, _SZ, _P], _I),
    "irb_sparse_gqa_attention_bwd_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "irb_sparse_gqa_attention_bwd_reads_out_f32": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, _I], _I),
    "irb_sparse_gqa_attention_bwd": ([_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                      _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P, _P], _I),
}
EXPORTED = tuple(_SIGS)

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libirb.so (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libirb.so not found at {path}; build it with indexer_routed_block_amd.build.build()")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def is_available() -> bool:
    return bool(load_library().irb_is_available())


def _check(status: int) -> None:
    if status == 0:
        return
    msg = load_library().irb_last_error().decode()
    if status == 2:
        raise TypeError(msg)
    if status == 3:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(*tensors) -> torch.device:
    """Device shared by every given tensor; it must be a GPU (no CPU path exists)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise RuntimeError(f"libirb runs on the GPU only; got a tensor on {t.device}")
        if dev is not None and t.device != dev:
            raise RuntimeError("all tensors must be on one device")
        dev = t.device
    return dev


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return IRB_BF16
    if t.dtype == torch.float32:
        return IRB_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t, name, dtype=None, contiguous=True, unit_last=False, shape=None):
    """Raise unless ``t`` (None passes) has the dtype, contiguity, last-axis
    stride and shape the C ABI assumes: the library receives bare pointers
    (and at most three strides), so it cannot check these itself."""
    if t is None:
        return
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if unit_last and t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous (stride 1)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


_ACT = (torch.bfloat16, torch.float32)
I32 = torch.int32


def make_layout(B: int, S: int, cu_seqlens: Optional[torch.Tensor] = None,
                row_lens: Optional[torch.Tensor] = None) -> IrbLayout:
    """Layout struct; ``num_docs`` comes from the host-side shape of cu_seqlens."""
    _req(cu_seqlens, "cu_seqlens", I32)
    _req(row_lens, "row_lens", I32, shape=None if row_lens is None else (B,))
    nd = 0 if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    return IrbLayout(B, S, None if cu_seqlens is None else cu_seqlens.data_ptr(), nd,
                     None if row_lens is None else row_lens.data_ptr())


def route_width(topk: int, c: int, window: int) -> int:
    """Fixed route width topk*c + max(window, c-1) (shape bookkeeping only)."""
    return topk * c + max(window, c - 1)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def compress_keys(k_idx, gamma, freqs, c, eps=1e-5, cu_seqlens=None, row_lens=None):
    """irb_compress_keys: returns (kc [B, S//c, D] fp32, cu_blocks or None)."""
    _gpu(k_idx, gamma, freqs, cu_seqlens, row_lens)
    lib = load_library()
    _req(k_idx, "k_idx", _ACT, contiguous=False, unit_last=True)
    _req(gamma, "gamma", torch.float32)
    _req(freqs, "freqs", torch.float32)
    B, S, D = k_idx.shape
    dev = k_idx.device
    kc = torch.empty((B, S // c, D), dtype=torch.float32, device=dev)
    cu_blocks = None if cu_seqlens is None else torch.empty(cu_seqlens.numel(), dtype=torch.int32, device=dev)
    lay = make_layout(B, S, cu_seqlens, row_lens)
    _check(lib.irb_compress_keys(ctypes.byref(lay), c, _ptr(k_idx), _dtype_code(k_idx), k_idx.stride(0),
                                 k_idx.stride(1), D, _ptr(gamma), eps, _ptr(freqs), freqs.shape[-1], _ptr(kc),
                                 _ptr(cu_blocks), _stream(dev)))
    return kc, cu_blocks


def prepare_index_queries(q_raw, gamma, freqs=None, eps=1e-5, out=None):
    """irb_prepare_index_queries: RMSNorm over the head dimension, then RoPE at each
    token's rotary row; q_raw [B, S, H, D] contiguous, freqs [B, S, D_rope] fp32
    (None: no rotation).  Returns [B, S, H, D] in q_raw's dtype (``out`` may be q_raw)."""
    _gpu(q_raw, gamma, freqs, out)
    lib = load_library()
    _req(q_raw, "q_raw", _ACT)
    _req(gamma, "gamma", torch.float32)
    _req(freqs, "freqs", torch.float32)
    _req(out, "out", q_raw.dtype, shape=q_raw.shape)
    B, S, H, D = q_raw.shape
    if out is None:
        out = torch.empty_like(q_raw)
    d_rope = 0 if freqs is None else freqs.shape[-1]
    _check(lib.irb_prepare_index_queries(_ptr(q_raw), _dtype_code(q_raw), B * S, H, D, _ptr(gamma), eps, _ptr(freqs),
                                         d_rope, _ptr(out), _stream(q_raw.device)))
    return out


def indexer_score_tile(q_idx, w, kc, c, q0=0, q1=None, j0=0, j1=None, score_scale=None, cu_blocks=None,
                       cu_seqlens=None, row_lens=None, out=None):
    """irb_indexer_score_tile: FP32 scores [B, q1-q0, j1-j0] (-inf where not visible).

    Index queries with a group axis, q_idx [B, S, R, H, D] and w [B, S, R, H],
    go to irb_indexer_score_tile_groups: scores [R, B, q1-q0, j1-j0]."""
    _gpu(q_idx, w, kc, cu_blocks, cu_seqlens, row_lens, out)
    lib = load_library()
    _req(q_idx, "q_idx", _ACT)
    _req(w, "w", torch.float32, shape=q_idx.shape[:-1])
    _req(kc, "kc", torch.float32)
    _req(cu_blocks, "cu_blocks", I32)
    _req(out, "out", torch.float32, contiguous=False, unit_last=True)
    grouped = q_idx.dim() == 5
    B, S, R, H, D = q_idx.shape if grouped else (q_idx.shape[0], q_idx.shape[1], 1, q_idx.shape[2], q_idx.shape[3])
    q1 = S if q1 is None else q1
    j1 = S // c if j1 is None else j1
    scale = 0.0 if score_scale is None else score_scale     # 0: the library's default 1/sqrt(D)
    if out is None:
        shape = (R, B, q1 - q0, j1 - j0) if grouped else (B, q1 - q0, j1 - j0)
        out = torch.empty(shape, dtype=torch.float32, device=q_idx.device)
    lay = make_layout(B, S, cu_seqlens, row_lens)
    if grouped:
        _check(lib.irb_indexer_score_tile_groups(ctypes.byref(lay), _ptr(q_idx), _dtype_code(q_idx), R, H, D, _ptr(w),
                                                 _ptr(kc), _ptr(cu_blocks), c, scale, q0, q1, j0, j1, _ptr(out),
                                                 out.stride(-2), _stream(q_idx.device)))
    else:
        _check(lib.irb_indexer_score_tile(ctypes.byref(lay), _ptr(q_idx), _dtype_code(q_idx), H, D, _ptr(w), _ptr(kc),
                                          _ptr(cu_blocks), c, scale, q0, q1, j0, j1, _ptr(out), out.stride(1),
                                          _stream(q_idx.device)))
    return out


def select_topk_regions(scores, c, topk, S, q0=0, cu_blocks=None, cu_seqlens=None, row_lens=None, sel=None,
                        cnt=None):
    """irb_select_topk_regions over score rows q0..q0+rows: (sel [B,S,topk], cnt [B,S])."""
    _gpu(scores, cu_blocks, cu_seqlens, row_lens, sel, cnt)
    lib = load_library()
    _req(scores, "scores", torch.float32, contiguous=False, unit_last=True)
    _req(cu_blocks, "cu_blocks", I32)
    B, rows, _ = scores.shape
    _req(sel, "sel", I32, shape=(B, S, topk))
    _req(cnt, "cnt", I32, shape=(B, S))
    dev = scores.device
    if sel is None:
        sel = torch.full((B, S, topk), -1, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.zeros((B, S), dtype=torch.int32, device=dev)
    lay = make_layout(B, S, cu_seqlens, row_lens)
    _check(lib.irb_select_topk_regions(ctypes.byref(lay), _ptr(scores), scores.stride(1), q0, q0 + rows,
                                       _ptr(cu_blocks), c, topk, _ptr(sel), _ptr(cnt), _stream(dev)))
    return sel, cnt


def route_topk_fused(q_idx, w, kc, c, topk, q0=0, q1=None, score_scale=None, cu_blocks=None, cu_seqlens=None,
                     row_lens=None, workspace=None, sel=None, cnt=None):
    """irb_route_topk_fused: scores and selection over bounded score chunks.

    Index queries with a group axis, q_idx [B, S, R, H, D] and w [B, S, R, H],
    go to irb_route_topk_fused_groups: sel [R, B, S, topk], cnt [R, B, S]."""
    _gpu(q_idx, w, kc, cu_blocks, cu_seqlens, row_lens, workspace, sel, cnt)
    lib = load_library()
    _req(q_idx, "q_idx", _ACT)
    _req(w, "w", torch.float32, shape=q_idx.shape[:-1])
    _req(kc, "kc", torch.float32)
    _req(cu_blocks, "cu_blocks", I32)
    _req(workspace, "workspace")
    grouped = q_idx.dim() == 5
    B, S, R, H, D = q_idx.shape if grouped else (q_idx.shape[0], q_idx.shape[1], 1, q_idx.shape[2], q_idx.shape[3])
    lead = (R,) if grouped else ()
    dev = q_idx.device
    q1 = S if q1 is None else q1
    scale = 0.0 if score_scale is None else score_scale     # 0: the library's default 1/sqrt(D)
    if workspace is None:
        n = (lib.irb_route_topk_fused_groups_workspace_size(B, S, c, D, topk, q0, q1, R) if grouped
             else lib.irb_route_topk_fused_workspace_size(B, S, c, D, topk, q0, q1))
        workspace = torch.empty(max(int(n), 4), dtype=torch.uint8, device=dev)
    if sel is None:
        sel = torch.full(lead + (B, S, topk), -1, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.zeros(lead + (B, S), dtype=torch.int32, device=dev)
    _req(sel, "sel", I32, shape=lead + (B, S, topk))
    _req(cnt, "cnt", I32, shape=lead + (B, S))
    lay = make_layout(B, S, cu_seqlens, row_lens)
    if grouped:
        _check(lib.irb_route_topk_fused_groups(ctypes.byref(lay), _ptr(q_idx), _dtype_code(q_idx), R, H, D, _ptr(w),
                                               _ptr(kc), _ptr(cu_blocks), c, scale, topk, q0, q1, _ptr(sel), _ptr(cnt),
                                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(dev)))
        return sel, cnt
    _check(lib.irb_route_topk_fused(ctypes.byref(lay), _ptr(q_idx), _dtype_code(q_idx), H, D, _ptr(w), _ptr(kc),
                                    _ptr(cu_blocks), c, scale, topk, q0, q1, _ptr(sel), _ptr(cnt), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(dev)))
    return sel, cnt


def route_topk_fused_raw(q_raw, gamma, freqs, w, kc, c, topk, eps=1e-5, q0=0, q1=None, score_scale=None,
                         cu_blocks=None, cu_seqlens=None, row_lens=None, workspace=None, sel=None, cnt=None):
    """irb_route_topk_fused_raw: route_topk_fused's selection from raw index queries
    q_raw [B, S, H, D], RMSNorm (gain ``gamma``) and RoPE (rows ``freqs`` [B, S, D_rope],
    None: no rotation) applied inside the score kernel."""
    _gpu(q_raw, gamma, freqs, w, kc, cu_blocks, cu_seqlens, row_lens, workspace, sel, cnt)
    lib = load_library()
    _req(q_raw, "q_raw", _ACT)
    _req(gamma, "gamma", torch.float32)
    _req(freqs, "freqs", torch.float32)
    _req(w, "w", torch.float32, shape=q_raw.shape[:-1])
    _req(kc, "kc", torch.float32)
    _req(cu_blocks, "cu_blocks", I32)
    _req(workspace, "workspace")
    B, S, H, D = q_raw.shape
    dev = q_raw.device
    q1 = S if q1 is None else q1
    scale = 0.0 if score_scale is None else score_scale
    if workspace is None:
        n = lib.irb_route_topk_fused_workspace_size(B, S, c, D, topk, q0, q1)
        workspace = torch.empty(max(int(n), 4), dtype=torch.uint8, device=dev)
    if sel is None:
        sel = torch.full((B, S, topk), -1, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.zeros((B, S), dtype=torch.int32, device=dev)
    _req(sel, "sel", I32, shape=(B, S, topk))
    _req(cnt, "cnt", I32, shape=(B, S))
    d_rope = 0 if freqs is None else freqs.shape[-1]
    lay = make_layout(B, S, cu_seqlens, row_lens)
    _check(lib.irb_route_topk_fused_raw(ctypes.byref(lay), _ptr(q_raw), _dtype_code(q_raw), H, D, _ptr(gamma), eps,
                                        _ptr(freqs), d_rope, _ptr(w), _ptr(kc), _ptr(cu_blocks), c, scale, topk, q0,
                                        q1, _ptr(sel), _ptr(cnt), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev)))
    return sel, cnt


def route_topk_fused_noalloc(q_idx, w, kc, c, topk, q0=0, q1=None, score_scale=None, cu_blocks=None,
                             cu_seqlens=None, row_lens=None, sel=None, cnt=None):
    """irb_route_topk_fused_noalloc: route_topk_fused's selection with the library's
    static per-device scratch instead of a workspace (the call allocates no device
    memory; pass ``sel`` / ``cnt`` to allocate nothing here either)."""
    _gpu(q_idx, w, kc, cu_blocks, cu_seqlens, row_lens, sel, cnt)
    lib = load_library()
    _req(q_idx, "q_idx", _ACT)
    _req(w, "w", torch.float32, shape=q_idx.shape[:-1])
    _req(kc, "kc", torch.float32)
    _req(cu_blocks, "cu_blocks", I32)
    B, S, H, D = q_idx.shape
    dev = q_idx.device
    q1 = S if q1 is None else q1
    scale = 0.0 if score_scale is None else score_scale
    if sel is None:
        sel = torch.full((B, S, topk), -1, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.zeros((B, S), dtype=torch.int32, device=dev)
    _req(sel, "sel", I32, shape=(B, S, topk))
    _req(cnt, "cnt", I32, shape=(B, S))
    lay = make_layout(B, S, cu_seqlens, row_lens)
    _check(lib.irb_route_topk_fused_noalloc(ctypes.byref(lay), _ptr(q_idx), _dtype_code(q_idx), H, D, _ptr(w), _ptr(kc),
                                            _ptr(cu_blocks), c, scale, topk, q0, q1, _ptr(sel), _ptr(cnt),
                                            _stream(dev)))
    return sel, cnt


def round_e4m3(x, out=None):
    """irb_round_e4m3: x (bf16 or fp32, contiguous) rounded to E4M3, stored as bf16 (``out`` may be a bf16 x)."""
    _gpu(x, out)
    lib = load_library()
    _req(x, "x", _ACT)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _req(out, "out", torch.bfloat16, shape=x.shape)
    _check(lib.irb_round_e4m3(_ptr(x), _dtype_code(x), x.numel(), _ptr(out), _stream(x.device)))
    return out


def gather_region_payload(keys, logits, sources, valid=None):
    """irb_gather_region_payload: (packed_keys, packed_logits) [B, R, region_size, D] in the keys' dtype."""
    _gpu(keys, logits, sources, valid)
    lib = load_library()
    _req(keys, "keys", _ACT)
    _req(logits, "logits", keys.dtype, shape=keys.shape)
    _req(sources, "sources", I32)
    if valid is not None:
        _req(valid, "valid", (torch.bool, torch.uint8), shape=sources.shape)
    B, T, D = keys.shape
    R, rs = sources.shape[1], sources.shape[2]
    pk = torch.empty((B, R, rs, D), dtype=keys.dtype, device=keys.device)
    pz = torch.empty_like(pk)
    _check(lib.irb_gather_region_payload(_ptr(keys), _ptr(logits), _dtype_code(keys), B, T, D, _ptr(sources),
                                         _ptr(valid), R, rs, _ptr(pk), _ptr(pz), _stream(keys.device)))
    return pk, pz


def summarize_region_payload(packed_keys, packed_logits, valid):
    """irb_summarize_region_payload: E4M3-rounded bf16 region summaries [B, R, D]."""
    _gpu(packed_keys, packed_logits, valid)
    lib = load_library()
    _req(packed_keys, "packed_keys", _ACT)
    _req(packed_logits, "packed_logits", packed_keys.dtype, shape=packed_keys.shape)
    _req(valid, "valid", (torch.bool, torch.uint8), shape=packed_keys.shape[:-1])
    B, R, rs, D = packed_keys.shape
    out = torch.empty((B, R, D), dtype=torch.bfloat16, device=packed_keys.device)
    _check(lib.irb_summarize_region_payload(_ptr(packed_keys), _ptr(packed_logits), _dtype_code(packed_keys),
                                            _ptr(valid), B, R, rs, D, _ptr(out), _stream(packed_keys.device)))
    return out


def select_regions_csa(scores, c, topk, S, q0=0, cu_blocks=None, cu_seqlens=None, row_lens=None, workspace=None):
    """irb_select_regions_csa over score rows q0..q0+rows: (region_ids [B, S, topk + 1], cnt [B, S])."""
    _gpu(scores, cu_blocks, cu_seqlens, row_lens, workspace)
    lib = load_library()
    _req(scores, "scores", torch.float32, contiguous=False, unit_last=True)
    _req(cu_blocks, "cu_blocks", I32)
    B, rows, _ = scores.shape
    dev = scores.device
    lay = make_layout(B, S, cu_seqlens, row_lens)
    if workspace is None:
        n = lib.irb_select_regions_csa_workspace_size(B, S, topk, lay.num_docs)
        workspace = torch.empty(max(int(n), 16), dtype=torch.uint8, device=dev)
    ids = torch.zeros((B, S, topk + 1), dtype=torch.int32, device=dev)
    cnt = torch.zeros((B, S), dtype=torch.int32, device=dev)
    _check(lib.irb_select_regions_csa(ctypes.byref(lay), _ptr(scores), scores.stride(1), q0, q0 + rows,
                                      _ptr(cu_blocks), c, topk, _ptr(ids), _ptr(cnt), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(dev)))
    return ids, cnt


def pack_region_bitmap(ids, regions, out=None):
    """irb_pack_region_bitmap: int32 membership words [..., ceil(regions / 32)] of int32 id rows [..., slots]."""
    _gpu(ids, out)
    lib = load_library()
    _req(ids, "ids", I32)
    slots = ids.shape[-1]
    rows = ids.numel() // max(slots, 1)
    words = (regions + 31) // 32
    if out is None:
        out = torch.empty(ids.shape[:-1] + (words,), dtype=torch.int32, device=ids.device)
    _req(out, "out", I32, shape=ids.shape[:-1] + (words,))
    _check(lib.irb_pack_region_bitmap(_ptr(ids), rows, slots, regions, _ptr(out), _stream(ids.device)))
    return out


def expand_and_compact_routes(sel, cnt, c, window, topk, L=None, cu_blocks=None, cu_seqlens=None, row_lens=None):
    """irb_expand_and_compact_routes: (routes [B,S,L] int32, lens [B,S] int32).

    Per-group selections sel [R, B, S, topk], cnt [R, B, S] expand group by
    group into routes [R, B, S, L], lens [R, B, S] (one call per group on
    its contiguous block)."""
    _gpu(sel, cnt, cu_blocks, cu_seqlens, row_lens)
    lib = load_library()
    _req(cnt, "cnt", I32)
    _req(sel, "sel", I32, shape=tuple(cnt.shape) + (topk,))
    _req(cu_blocks, "cu_blocks", I32)
    lead = tuple(cnt.shape[:-2])
    B, S = cnt.shape[-2:]
    dev = cnt.device
    L = route_width(topk, c, window) if L is None else L
    routes = torch.empty(lead + (B, S, L), dtype=torch.int32, device=dev)
    lens = torch.empty(lead + (B, S), dtype=torch.int32, device=dev)
    lay = make_layout(B, S, cu_seqlens, row_lens)
    R = lead[0] if lead else 1
    sel_g = sel.reshape(R, B, S, topk)
    cnt_g = cnt.reshape(R, B, S)
    r_g, l_g = routes.view(R, B, S, L), lens.view(R, B, S)
    for g in range(R):
        _check(lib.irb_expand_and_compact_routes(ctypes.byref(lay), _ptr(sel_g[g]), _ptr(cnt_g[g]), topk, c, window,
                                                 _ptr(cu_blocks), L, _ptr(r_g[g]), _ptr(l_g[g]), _stream(dev)))
    return routes, lens


def compact_routes(ids, key_count, out=None, count_out_of_range=True):
    """irb_compact_routes over the last axis: (ids_out, lens, out_of_range counter or None)."""
    _gpu(ids, out)
    lib = load_library()
    _req(ids, "ids", I32)
    _req(out, "out", I32, shape=ids.shape)
    width = ids.shape[-1]
    rows = ids.numel() // width
    dev = ids.device
    out = torch.empty_like(ids) if out is None else out
    lens = torch.empty(ids.shape[:-1], dtype=torch.int32, device=dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev) if count_out_of_range else None
    _check(lib.irb_compact_routes(_ptr(ids), rows, width, key_count, _ptr(out), _ptr(lens), _ptr(bad), _stream(dev)))
    return out, lens, bad


def build_block_lists(routes, lens, S_k, block_q, block_k, reverse, width=None, workspace=None):
    """irb_build_block_lists: (counts [B, rows], indices [B, rows, width]).

    Per-group routes [R, B, S_q, L] are R * B route rows: counts [R, B, rows],
    indices [R, B, rows, width]."""
    _gpu(routes, lens, workspace)
    lib = load_library()
    _req(routes, "routes", I32)
    _req(lens, "lens", I32, shape=routes.shape[:-1])
    _req(workspace, "workspace")
    lead = tuple(routes.shape[:-3])
    B, S_q, L = routes.shape[-3:]
    B_all = B * (lead[0] if lead else 1)
    dev = routes.device
    nqt, nkt = -(-S_q // block_q), -(-S_k // block_k)
    rows, other = (nkt, nqt) if reverse else (nqt, nkt)
    width = other if width is None else width
    if workspace is None:
        n = lib.irb_build_block_lists_workspace_size(B_all, S_q, S_k, block_q, block_k)
        workspace = torch.empty(max(int(n), 4), dtype=torch.uint8, device=dev)
    counts = torch.empty(lead + (B, rows), dtype=torch.int32, device=dev)
    indices = torch.empty(lead + (B, rows, width), dtype=torch.int32, device=dev)
    _check(lib.irb_build_block_lists(_ptr(routes), _ptr(lens), B_all, S_q, S_k, L, block_q, block_k, int(bool(reverse)),
                                     _ptr(counts), _ptr(indices), width, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(dev)))
    return counts, indices


def split_full_blocks(routes, lens, S_k, block_q, block_k, reverse, counts, indices, workspace=None,
                      use_workspace=True):
    """irb_split_full_blocks: (full_counts, full_indices, part_counts, part_indices) in the lists' layout.

    Index entries past each count are left unwritten (uninitialised memory).
    With one-query tiles a coverage-bit workspace is allocated unless
    ``use_workspace`` is False (then every pair searches its route)."""
    _gpu(routes, lens, counts, indices)
    lib = load_library()
    _req(routes, "routes", I32)
    _req(lens, "lens", I32, shape=routes.shape[:-1])
    _req(counts, "counts", I32)
    _req(indices, "indices", I32)
    lead = tuple(routes.shape[:-3])
    B, S_q, L = routes.shape[-3:]
    B_all = B * (lead[0] if lead else 1)
    width = indices.shape[-1]
    fc, pc = torch.empty_like(counts), torch.empty_like(counts)
    fi, pi = torch.empty_like(indices), torch.empty_like(indices)
    if workspace is None and use_workspace:
        n = lib.irb_split_full_blocks_workspace_size(B_all, S_q, S_k, block_q, block_k)
        workspace = torch.empty(int(n), dtype=torch.uint8, device=routes.device) if n > 0 else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.irb_split_full_blocks(_ptr(routes), _ptr(lens), B_all, S_q, S_k, L, block_q, block_k, int(bool(reverse)),
                                     _ptr(counts), _ptr(indices), width, _ptr(fc), _ptr(fi), _ptr(pc), _ptr(pi),
                                     _ptr(workspace), ws_bytes, _stream(routes.device)))
    return fc, fi, pc, pi


def _strides9(q, k, v):
    return (ctypes.c_int64 * 9)(q.stride(0), q.stride(1), q.stride(2), k.stride(0), k.stride(1), k.stride(2),
                                v.stride(0), v.stride(1), v.stride(2))


def _check_qkv(q, k, v, routes, lens):
    """q / k / v: one activation dtype, 4-D, last dimension contiguous (other
    strides are passed); routes / lens: contiguous int32 of matching shapes."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, n, q.dtype if n != "q" else _ACT, contiguous=False, unit_last=True)
        if t.dim() != 4:
            raise ValueError(f"{n}: expected [B, S, H, D], got shape {tuple(t.shape)}")
    if k.shape[:3] != v.shape[:3] or k.shape[0] != q.shape[0]:
        raise ValueError("k and v must share [B, S_k, Hkv], and B must match q")
    _req(routes, "routes", I32)
    _req(lens, "lens", I32, shape=routes.shape[:-1])
    if routes.shape[-2] != q.shape[1] or routes.shape[-3] != q.shape[0]:
        raise ValueError(f"routes {tuple(routes.shape)} do not match q's [B, S_q] {tuple(q.shape[:2])}")


def _route_groups(routes, lens):
    """Route groups of a routes tensor: [B, S, L] -> 1, [RG, B, S, L] (per KV group) -> RG."""
    if routes.dim() == 4:
        if lens.dim() != 3 or tuple(lens.shape) != tuple(routes.shape[:3]):
            raise ValueError("grouped routes [RG, B, S, L] need lens [RG, B, S]")
        return routes.shape[0]
    return 1


def sparse_gqa_attention_fwd(q, k, v, routes, lens, softmax_scale=None, out=None, lse=None, workspace=None,
                             use_workspace=True, out_f32=None):
    """irb_sparse_gqa_attention_fwd: (o [B,S_q,Hq,Dv] in q's dtype, lse [B,Hq,S_q] fp32).

    routes [B, S_q, L] are shared by every head; routes [Hkv, B, S_q, L]
    (lens [Hkv, B, S_q]) give every KV group its own routes.  The
    key-membership workspace is allocated here unless given or
    ``use_workspace`` is False (then the query tiles build their masks in LDS).
    ``out_f32`` (True, or an fp32 tensor of o's shape) also writes o before
    its rounding, the backward's Delta input; the result is then (o, lse, o32)."""
    _gpu(q, k, v, routes, lens, out, lse, workspace)
    lib = load_library()
    _check_qkv(q, k, v, routes, lens)
    B, S_q, Hq, Dqk = q.shape
    S_k, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    dev = q.device
    scale = 0.0 if softmax_scale is None else softmax_scale     # 0: the library's default 1/sqrt(Dqk)
    if out is None:
        out = torch.empty((B, S_q, Hq, Dv), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=dev)
    _req(out, "out", q.dtype, shape=(B, S_q, Hq, Dv))
    _req(lse, "lse", torch.float32, shape=(B, Hq, S_q))
    if out_f32 is True:
        out_f32 = torch.empty((B, S_q, Hq, Dv), dtype=torch.float32, device=dev)
    elif out_f32 is not None:
        _gpu(out_f32)
        _req(out_f32, "out_f32", torch.float32, shape=(B, S_q, Hq, Dv))
    rg = _route_groups(routes, lens)
    if workspace is None and use_workspace:
        n = lib.irb_sparse_gqa_attention_fwd_workspace_size(B, S_q, S_k, routes.shape[-1], Hq, Hkv, Dqk, Dv,
                                                            _dtype_code(q), rg)
        workspace = torch.empty(int(n), dtype=torch.uint8, device=dev) if n > 0 else None
    _req(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.irb_sparse_gqa_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _strides9(q, k, v),
                                            _ptr(routes), _ptr(lens), rg, B, S_q, S_k,
                                            routes.shape[-1], Hq, Hkv, Dqk, Dv, scale, _ptr(out), _ptr(lse),
                                            _ptr(out_f32), _ptr(workspace), ws_bytes, _stream(dev)))
    return (out, lse) if out_f32 is None else (out, lse, out_f32)


def sparse_gqa_attention_bwd(q, k, v, out, dout, lse, routes, lens, rev_counts, rev_indices, rev_block_q,
                             rev_block_k=16, softmax_scale=None, merged_kv=False, workspace=None, dropped_hits=None,
                             out_f32=None):
    """irb_sparse_gqa_attention_bwd: (dq, dk, dv); with merged_kv (v aliases k) dk holds dK + [dV, 0], dv is dk.

    ``out`` (the forward's output in q's dtype) is not read: Delta comes from
    ``out_f32`` (the forward's FP32 output, optional) or is formed from the
    routes.

    ``dropped_hits`` (int64 [1] on the device, optional) receives the number of
    key-side hit entries that did not fit the workspace (0 for reverse lists
    built from the same routes).

    Grouped routes [Hkv, B, S_q, L] take the reverse lists of the routes
    viewed as Hkv * B rows."""
    _gpu(q, k, v, out, dout, lse, routes, lens, rev_counts, rev_indices, workspace, dropped_hits)
    lib = load_library()
    _check_qkv(q, k, v, routes, lens)
    B, S_q, Hq, Dqk = q.shape
    S_k, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    dev = q.device
    _req(dout, "dout", q.dtype, shape=(B, S_q, Hq, Dv))
    _req(lse, "lse", torch.float32, shape=(B, Hq, S_q))
    if out_f32 is not None:
        _gpu(out_f32)
        _req(out_f32, "out_f32", torch.float32, shape=(B, S_q, Hq, Dv))
    _req(rev_counts, "rev_counts", I32)
    _req(rev_indices, "rev_indices", I32)
    _req(workspace, "workspace")
    _req(dropped_hits, "dropped_hits", torch.int64, shape=(1,))
    scale = 0.0 if softmax_scale is None else softmax_scale     # 0: the library's default 1/sqrt(Dqk)
    dq = torch.empty((B, S_q, Hq, Dqk), dtype=q.dtype, device=dev)
    dk = torch.empty((B, S_k, Hkv, Dqk), dtype=q.dtype, device=dev)
    dv = dk if merged_kv else torch.empty((B, S_k, Hkv, Dv), dtype=q.dtype, device=dev)
    rg = _route_groups(routes, lens)
    if rg not in (1, Hkv):
        raise ValueError(f"sparse_gqa_attention_bwd: {rg} route groups for {Hkv} KV heads")
    nkt = -(-S_k // rev_block_k)
    if rev_counts.numel() != rg * B * nkt or rev_indices.numel() != rg * B * nkt * rev_indices.shape[-1]:
        raise ValueError("sparse_gqa_attention_bwd: reverse lists do not match the routes "
                         f"({rg} groups x {B} rows x {nkt} key tiles)")
    if workspace is None:
        n = lib.irb_sparse_gqa_attention_bwd_workspace_size(B, S_q, S_k, routes.shape[-1], Hq, Hkv, Dqk, Dv,
                                                            _dtype_code(q), rg)
        workspace = torch.empty(max(int(n), 4), dtype=torch.uint8, device=dev)
    _check(lib.irb_sparse_gqa_attention_bwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _strides9(q, k, v), _ptr(out_f32), _ptr(dout), _ptr(lse),
        _ptr(routes), _ptr(lens), rg, _ptr(rev_counts), _ptr(rev_indices), rev_block_q, rev_block_k,
        rev_indices.shape[-1], B, S_q, S_k, routes.shape[-1], Hq, Hkv, Dqk, Dv, scale, _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(dropped_hits), _stream(dev)))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# composition of the entry points (host scalars only; no device reads)
# ---------------------------------------------------------------------------

def first_sparse_query(c: int, topk: int) -> int:
    """First document position whose query sees more than topk complete blocks."""
    return (topk + 1) * c - 1


def route(k_idx, q_idx, w, gamma, freqs, c, topk, window, eps=1e-5, score_scale=None, cu_seqlens=None,
          row_lens=None, workspace=None):
    """compress -> fused score/select -> expand, all in the library.

    Returns dict(kc, cu_blocks, sel, cnt, routes, lens).  Query rows that see
    at most topk blocks take every visible block: the fused call does not
    score them and its selection takes them without scores.  Index queries with a group axis
    (q_idx [B, S, R, H, D], w [B, S, R, H]) give every group its own
    selection and routes: sel [R, B, S, topk], routes [R, B, S, L].
    """
    B, S = q_idx.shape[:2]
    grouped = q_idx.dim() == 5
    R = q_idx.shape[2] if grouped else 1
    lead = (R,) if grouped else ()
    kc, cu_blocks = compress_keys(k_idx, gamma, freqs, c, eps, cu_seqlens, row_lens)
    sel = torch.empty(lead + (B, S, topk), dtype=torch.int32, device=q_idx.device)
    cnt = torch.empty(lead + (B, S), dtype=torch.int32, device=q_idx.device)
    route_topk_fused(q_idx, w, kc, c, topk, q0=0, q1=S, score_scale=score_scale, cu_blocks=cu_blocks,
                     cu_seqlens=cu_seqlens, row_lens=row_lens, workspace=workspace, sel=sel, cnt=cnt)
    routes, lens = expand_and_compact_routes(sel, cnt, c, window, topk, cu_blocks=cu_blocks, cu_seqlens=cu_seqlens,
                                             row_lens=row_lens)
    return dict(kc=kc, cu_blocks=cu_blocks, sel=sel, cnt=cnt, routes=routes, lens=lens)
