"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host (no GPU needed: validation runs before any
device call, and nothing here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import indexer_routed_block_amd as irb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "irb.h")

pytestmark = pytest.mark.skipif(not os.path.exists(irb.LIB_PATH), reason="libirb.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(irb_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = irb.load_library()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(irb.EXPORTED) == names


def test_version_and_availability_without_gpu():
    lib = irb.load_library()
    assert b"gfx950" in lib.irb_version()
    assert lib.irb_is_available() in (0, 1)


def _layout(B=1, S=64, cu=None, nd=0, rl=None):
    return irb.IrbLayout(B, S, cu, nd, rl)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _err(status):
    return status, irb.load_library().irb_last_error().decode()


def test_compress_keys_validation():
    lib = irb.load_library()
    lay = _layout()
    s, m = _err(lib.irb_compress_keys(None, 4, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, None, None))
    assert s == 3 and "layout" in m
    s, m = _err(lib.irb_compress_keys(ctypes.byref(lay), 4, FAKE, 7, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, None, None))
    assert s == 2
    s, m = _err(lib.irb_compress_keys(ctypes.byref(lay), 0, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, None, None))
    assert s == 3 and "c must" in m
    s, m = _err(lib.irb_compress_keys(ctypes.byref(lay), 4, FAKE, 1, 0, 64, 48, FAKE, 1e-5, FAKE, 48, FAKE, None, None))
    assert s == 3 and "D_idx" in m
    s, m = _err(lib.irb_compress_keys(ctypes.byref(lay), 4, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 63, FAKE, None, None))
    assert s == 3 and "D_rope" in m
    packed = _layout(cu=0x2000, nd=3)
    s, m = _err(lib.irb_compress_keys(ctypes.byref(packed), 4, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, None, None))
    assert s == 3 and "cu_blocks" in m
    both = _layout(cu=0x2000, nd=3, rl=0x3000)
    s, m = _err(lib.irb_compress_keys(ctypes.byref(both), 4, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, FAKE, None))
    assert s == 3 and "not both" in m
    batched_packed = _layout(B=2, cu=0x2000, nd=3)
    s, m = _err(lib.irb_compress_keys(ctypes.byref(batched_packed), 4, FAKE, 1, 0, 64, 64, FAKE, 1e-5, FAKE, 64, FAKE, FAKE, None))
    assert s == 3 and "B == 1" in m


def test_score_and_select_validation():
    lib = irb.load_library()
    lay = _layout(S=64)
    args = lambda H=16, D=128, sc=0.1, q0=0, q1=64, j0=0, j1=16, st=16: lib.irb_indexer_score_tile(
        ctypes.byref(lay), FAKE, 1, H, D, FAKE, FAKE, None, 4, sc, q0, q1, j0, j1, FAKE, st, None)
    assert _err(args(H=12))[0] == 3
    assert _err(args(D=96))[0] == 3
    assert _err(args(sc=-0.5))[0] == 3
    assert _err(args(sc=float("nan")))[0] == 3
    assert _err(args(sc=0.0))[0] == 1      # 0 = default 1/sqrt(D_idx): valid; no GPU here
    assert _err(args(q0=10, q1=10))[0] == 3
    assert _err(args(j1=17))[0] == 3
    assert _err(args(st=8))[0] == 3
    s = lib.irb_select_topk_regions(ctypes.byref(lay), FAKE, 16, 0, 64, None, 4, 0, FAKE, FAKE, None)
    assert _err(s)[0] == 3
    s = lib.irb_select_topk_regions(ctypes.byref(lay), FAKE, 16, 0, 65, None, 4, 4, FAKE, FAKE, None)
    assert _err(s)[0] == 3


def test_routes_lists_validation():
    lib = irb.load_library()
    lay = _layout(S=64)
    # width below topk*c + max(window, c-1)
    s, m = _err(lib.irb_expand_and_compact_routes(ctypes.byref(lay), FAKE, FAKE, 4, 4, 8, None, 23, FAKE, FAKE, None))
    assert s == 3 and "width" in m
    s, m = _err(lib.irb_compact_routes(FAKE, 4, 0, 10, FAKE, FAKE, None, None))
    assert s == 3
    s, m = _err(lib.irb_compact_routes(FAKE, 4, 8, 0, FAKE, FAKE, None, None))
    assert s == 3
    need = lib.irb_build_block_lists_workspace_size(1, 64, 64, 16, 16)
    assert need == 4 * 4
    s, m = _err(lib.irb_build_block_lists(FAKE, FAKE, 1, 64, 64, 8, 16, 16, 0, FAKE, FAKE, 3, FAKE, need, None))
    assert s == 3 and "width" in m
    s, m = _err(lib.irb_build_block_lists(FAKE, FAKE, 1, 64, 64, 8, 16, 16, 0, FAKE, FAKE, 4, FAKE, need - 1, None))
    assert s == 3 and "workspace" in m


def test_split_full_blocks_validation():
    lib = irb.load_library()
    A, B_, C_, D_, E_ = (ctypes.c_void_p(0x1000 * k) for k in range(1, 6))
    call = lambda bq=16, bk=16, width=8, fi=C_, pi=D_, fc=E_, pc=ctypes.c_void_p(0x7000): lib.irb_split_full_blocks(
        A, B_, 1, 64, 64, 8, bq, bk, 0, ctypes.c_void_p(0x9000), ctypes.c_void_p(0xA000), width, fc, fi, pc, pi, None,
        0, None)
    assert _err(call(bq=0))[0] == 3
    assert _err(call(width=0))[0] == 3
    code, msg = _err(call(fi=ctypes.c_void_p(0xA000)))
    assert code == 3 and "alias" in msg
    assert _err(call(fi=D_))[0] == 3
    assert _err(call(pc=E_))[0] == 3
    # coverage bits: one-query tiles only, one bit per (query, key tile), rows of 32-bit words
    assert lib.irb_split_full_blocks_workspace_size(2, 100, 1000, 1, 16) == 2 * 100 * 2 * 4
    assert lib.irb_split_full_blocks_workspace_size(2, 100, 1000, 4, 16) == 0


def test_grouped_route_workspace_size():
    lib = irb.load_library()
    one = lib.irb_route_topk_fused_workspace_size(1, 8192, 4, 128, 512, 2044, 8192)
    four = lib.irb_route_topk_fused_groups_workspace_size(1, 8192, 4, 128, 512, 2044, 8192, 4)
    split = 8192 // 4 * 128 * 4          # the split keys, held once
    assert four - split == 4 * (one - split)
    assert lib.irb_route_topk_fused_groups_workspace_size(1, 8192, 4, 128, 512, 2044, 8192, 1) == one
    assert lib.irb_route_topk_fused_groups_workspace_size(1, 8192, 4, 128, 512, 2044, 8192, 0) == 0
    assert lib.irb_route_topk_fused_groups_workspace_size(1, 8192, 4, 128, 512, 2044, 8192, 65) == 0


def test_attention_validation():
    lib = irb.load_library()
    st = (ctypes.c_int64 * 9)(64 * 4 * 128, 4 * 128, 128, 64 * 128, 128, 128, 64 * 128, 128, 128)
    call = lambda Hq=4, Hkv=1, D=128, Dv=128, sc=0.1, dt=1, strides=st, rg=1: lib.irb_sparse_gqa_attention_fwd(
        FAKE, FAKE, FAKE, dt, strides, FAKE, FAKE, rg, 1, 64, 64, 16, Hq, Hkv, D, Dv, sc, FAKE, FAKE, None, None, 0,
        None)
    assert _err(call(Hq=6, Hkv=4))[0] == 3
    assert _err(call(Hq=128, Hkv=1))[0] == 3
    assert _err(call(D=96, Dv=96))[0] == 3
    assert _err(call(D=576, Dv=512, dt=0))[0] == 3      # latent dims are bf16 only
    assert _err(call(sc=-1.0))[0] == 3
    assert _err(call(sc=float("nan")))[0] == 3
    assert _err(call(sc=float("inf")))[0] == 3
    # 0 selects the default 1/sqrt(Dqk): validation passes, and with no GPU here the call stops at the device check
    assert _err(call(sc=0.0))[0] == 1
    assert _err(call(dt=5))[0] == 2
    odd = (ctypes.c_int64 * 9)(*list(st)[:8], 129)
    assert _err(call(strides=odd))[0] == 3
    # forward workspace: key-membership words of every route row where the query-tile kernel runs
    fws = lib.irb_sparse_gqa_attention_fwd_workspace_size
    assert fws(1, 8192, 8192, 2176, 32, 4, 128, 128, 1, 1) == 8192 * 256 * 4
    assert fws(1, 8192, 8192, 2176, 32, 4, 128, 128, 1, 4) == 4 * 8192 * 256 * 4
    assert fws(1, 8192, 8192, 2176, 32, 4, 128, 128, 0, 1) == 0          # fp32: no query-tile kernel
    assert fws(1, 16384, 16384, 2048, 64, 1, 576, 512, 1, 1) == 0        # latent rows
    assert fws(1, 131072, 131072, 2560, 64, 8, 128, 128, 1, 1) == 0      # 2 GiB of words: over the budget
    misaligned = lambda: lib.irb_sparse_gqa_attention_fwd(FAKE, FAKE, FAKE, 1, st, FAKE, FAKE, 1, 1, 64, 64, 16, 4, 1,
                                                          128, 128, 0.1, FAKE, FAKE, None, ctypes.c_void_p(0x1004),
                                                          64, None)
    assert _err(misaligned())[0] == 3
    # the optional FP32 output must be 16-byte aligned (forward and backward)
    o32_bad = lambda: lib.irb_sparse_gqa_attention_fwd(FAKE, FAKE, FAKE, 1, st, FAKE, FAKE, 1, 1, 64, 64, 16, 4, 1,
                                                       128, 128, 0.1, FAKE, FAKE, ctypes.c_void_p(0x1004), None, 0,
                                                       None)
    code, msg = _err(o32_bad())
    assert code == 3 and "out_f32" in msg
    # empty sizes are rejected before anything is enqueued
    sized = lambda B=1, S_q=64, S_k=64, L=16: lib.irb_sparse_gqa_attention_fwd(
        FAKE, FAKE, FAKE, 1, st, FAKE, FAKE, 1, B, S_q, S_k, L, 4, 1, 128, 128, 0.1, FAKE, FAKE, None, None, 0, None)
    for kw in ({"B": 0}, {"S_q": 0}, {"S_k": 0}, {"L": 0}):
        code, msg = _err(sized(**kw))
        assert code == 3 and "sizes" in msg, kw
    # route groups: 1 (shared) or one per KV head
    code, msg = _err(call(Hq=8, Hkv=4, rg=2))
    assert code == 3 and "route_groups" in msg
    assert _err(call(Hq=8, Hkv=4, rg=0))[0] == 3
    # backward: key tile must be 16, merged dk/dv needs Dv <= Dqk
    bwd = lambda bk=16, width=64, ws=1 << 30, rg=1: lib.irb_sparse_gqa_attention_bwd(
        FAKE, FAKE, FAKE, 1, st, FAKE, FAKE, FAKE, FAKE, FAKE, rg, FAKE, FAKE, 1, bk, width, 1, 64, 64, 16, 4, 1, 128,
        128, 0.1, FAKE, FAKE, FAKE, FAKE, ws, None, None)
    assert _err(bwd(bk=32))[0] == 3
    code, msg = _err(lib.irb_sparse_gqa_attention_bwd(
        FAKE, FAKE, FAKE, 1, st, ctypes.c_void_p(0x1004), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, 16, 64, 1, 64, 64,
        16, 4, 1, 128, 128, 0.1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None))
    assert code == 3 and "out_f32" in msg
    assert _err(bwd(width=63))[0] == 3
    assert _err(bwd(rg=2))[0] == 3
    need = lib.irb_sparse_gqa_attention_bwd_workspace_size(1, 64, 64, 16, 4, 1, 128, 128, 1, 1)
    assert need > 0
    code, msg = _err(bwd(ws=need - 1))
    assert code == 3 and "workspace" in msg
    assert lib.irb_sparse_gqa_attention_bwd_workspace_size(1, 64, 64, 16, 6, 4, 128, 128, 1, 1) == 0
    # the hit lists of the bf16 GQA path grow with the route width and the route groups; fp32 keeps the
    # transposed copies
    ws_size = lib.irb_sparse_gqa_attention_bwd_workspace_size
    assert ws_size(1, 256, 256, 16, 4, 1, 128, 128, 1, 1) > ws_size(1, 256, 256, 8, 4, 1, 128, 128, 1, 1)
    assert ws_size(1, 256, 256, 16, 8, 4, 128, 128, 1, 4) > ws_size(1, 256, 256, 16, 8, 4, 128, 128, 1, 1)
    assert ws_size(1, 256, 256, 16, 8, 4, 128, 128, 1, 3) == 0
    assert lib.irb_sparse_gqa_attention_bwd_workspace_size(1, 64, 64, 16, 4, 1, 128, 128, 0, 1) != need
    # where the backward reads Delta off the forward's FP32 output
    reads = lib.irb_sparse_gqa_attention_bwd_reads_out_f32
    assert reads(1, 32768, 32768, 1024, 32, 4, 128, 128, 1, 1) == 1      # packed 32768: query-tile dQ
    assert reads(1, 131072, 131072, 2560, 64, 8, 128, 128, 1, 1) == 0    # per-query dQ forms Delta itself
    assert reads(1, 16384, 16384, 2048, 64, 1, 576, 512, 1, 1) == 1      # latent rows
    assert reads(1, 512, 512, 64, 4, 1, 64, 64, 0, 1) == 1               # fp32: Delta-mode forward saved
    assert reads(1, 300, 300, 96, 32, 1, 128, 128, 1, 1) == 1            # 32 heads per group: the same
    assert reads(1, 64, 64, 16, 6, 4, 128, 128, 1, 1) == 0               # invalid head counts


def test_python_binding_has_no_cpu_path():
    import torch
    x = torch.zeros(1, 64, 64)
    with pytest.raises(RuntimeError, match="GPU only"):
        irb.compress_keys(x, torch.ones(64), torch.zeros(1, 64, 64), 4)
    q = torch.zeros(1, 8, 2, 64)
    r = torch.zeros(1, 8, 4, dtype=torch.int32)
    with pytest.raises(RuntimeError, match="GPU only"):
        irb.sparse_gqa_attention_fwd(q, q[:, :, :1], q[:, :, :1], r, r[..., 0])


def test_prepare_index_queries_validation():
    lib = irb.load_library()
    call = lambda q=FAKE, dt=1, n=10, H=4, D=128, g=FAKE, eps=1e-5, r=FAKE, R=128, o=FAKE: _err(
        lib.irb_prepare_index_queries(q, dt, n, H, D, g, eps, r, R, o, None))
    s, m = call(dt=7)
    assert s == 2
    s, m = call(D=48)
    assert s == 3 and "D_idx" in m
    s, m = call(R=7)
    assert s == 3 and "D_rope" in m
    s, m = call(R=256)
    assert s == 3 and "D_rope" in m
    s, m = call(q=None)
    assert s == 3 and "NULL" in m
    s, m = call(r=None)
    assert s == 3 and "NULL" in m
    s, m = call(o=ctypes.c_void_p(0x1008))
    assert s == 3 and "aligned" in m
    s, m = call(eps=-1.0)
    assert s == 3 and "eps" in m
    s, m = call(H=0)
    assert s == 3
    assert call(n=0)[0] == 0          # nothing to do: no device call


def test_route_raw_validation():
    """The fused-preparation route checks the preparation arguments on the host
    before the route arguments; a valid call stops at the device check."""
    lib = irb.load_library()
    lay = _layout(S=8192)
    call = lambda g=FAKE, eps=1e-5, r=FAKE, R=128, D=128: _err(lib.irb_route_topk_fused_raw(
        ctypes.byref(lay), FAKE, 1, 16, D, g, eps, r, R, FAKE, FAKE, None, 4, 0.0, 512, 0, 8192, FAKE, FAKE, FAKE,
        1 << 24, None))
    s, m = call(g=None)
    assert s == 3 and "gamma" in m
    s, m = call(g=ctypes.c_void_p(0x1004))
    assert s == 3 and "gamma" in m
    s, m = call(eps=-1.0)
    assert s == 3 and "eps" in m
    for R in (32, 96, 256):              # not a multiple of 64 up to D_idx
        s, m = call(R=R)
        assert s == 3 and "D_rope" in m
    s, m = call(R=128, D=64)
    assert s == 3 and "D_rope" in m
    s, m = call(r=None)
    assert s == 3 and "rope" in m
    s, m = call(r=ctypes.c_void_p(0x1008))
    assert s == 3 and "rope" in m
    assert call()[0] == 1                # valid: stops at the device check (no GPU here)
    assert call(r=None, R=0)[0] == 1     # no rotation: the table is not needed
    assert call(R=64)[0] == 1            # partial rotation


def test_pack_region_bitmap_validation():
    lib = irb.load_library()
    call = lambda ids=FAKE, rows=4, slots=8, regions=100, out=FAKE: _err(
        lib.irb_pack_region_bitmap(ids, rows, slots, regions, out, None))
    s, m = call(slots=0)
    assert s == 3 and "slots" in m
    s, m = call(regions=0)
    assert s == 3 and "regions" in m
    s, m = call(regions=131073)
    assert s == 3 and "regions" in m
    s, m = call(ids=None)
    assert s == 3 and "NULL" in m
    s, m = call(rows=-1)
    assert s == 3
    assert call(rows=0, ids=None, out=None)[0] == 0      # nothing to do: no device call


def test_binding_rejects_layouts_the_abi_cannot_see():
    """dtype, contiguity, unit last stride and shapes are checked in the binding
    (the C ABI receives bare pointers); CPU tensors exercise the checks alone."""
    import torch
    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    r = torch.zeros(1, 8, 16, dtype=torch.int32)
    n = torch.zeros(1, 8, dtype=torch.int32)
    irb._check_qkv(q, k, k, r, n)                                     # well formed
    with pytest.raises(TypeError, match="routes"):
        irb._check_qkv(q, k, k, r.long(), n)                          # int64 ids (torch.topk's default)
    with pytest.raises(ValueError, match="routes"):
        irb._check_qkv(q, k, k, r[..., ::2], n)                       # strided ids
    with pytest.raises(ValueError, match="lens"):
        irb._check_qkv(q, k, k, r, n[:, :4])
    with pytest.raises(ValueError, match="last dimension"):
        irb._check_qkv(q, k[..., ::2], k[..., ::2], r, n)
    with pytest.raises(TypeError, match="k"):
        irb._check_qkv(q, k.float(), k, r, n)
    with pytest.raises(ValueError, match="do not match"):
        irb._check_qkv(q, k, k, r[:, :4], n[:, :4])
    # an expanded gradient (stride 0, e.g. the gradient of o.sum()) is not contiguous
    dout = torch.zeros(1, dtype=torch.bfloat16).expand(1, 8, 4, 64)
    with pytest.raises(ValueError, match="contiguous"):
        irb._req(dout, "dout", torch.bfloat16, shape=(1, 8, 4, 64))
    with pytest.raises(ValueError, match="shape"):
        irb._req(torch.zeros(1, 4, 8), "lse", torch.float32, shape=(1, 4, 9))


def test_noalloc_route_rejects_inputs_beyond_its_scratch():
    """The allocation-free fused route checks its static scratch bound on the host
    (no device needed): 2^20 blocks of 128 dims need 512 MiB of split keys."""
    lib = irb.load_library()
    big = _layout(S=1 << 22)
    code, msg = _err(lib.irb_route_topk_fused_noalloc(ctypes.byref(big), FAKE, 1, 16, 128, FAKE, FAKE, None, 4, 0.0,
                                                      512, 0, 1 << 22, FAKE, FAKE, None))
    assert code == 3 and "static maximum" in msg
    ok = _layout(S=8192)
    # within the bound: validation passes and the call stops at the device check (no GPU here)
    assert _err(lib.irb_route_topk_fused_noalloc(ctypes.byref(ok), FAKE, 1, 16, 128, FAKE, FAKE, None, 4, 0.0, 512,
                                                 0, 8192, FAKE, FAKE, None))[0] == 1
    assert _err(lib.irb_route_topk_fused_noalloc(ctypes.byref(ok), FAKE, 1, 12, 128, FAKE, FAKE, None, 4, 0.0, 512,
                                                 0, 8192, FAKE, FAKE, None))[0] == 3


def test_csa_validation():
    lib = irb.load_library()
    # E4M3 rounding: dtype, n
    assert _err(lib.irb_round_e4m3(FAKE, 7, 10, FAKE, None))[0] == 2
    assert _err(lib.irb_round_e4m3(FAKE, 1, -1, FAKE, None))[0] == 3
    assert _err(lib.irb_round_e4m3(None, 1, 0, None, None))[0] == 0          # nothing to do
    # payload gather: rows must be whole 16-byte pieces, pointers aligned
    s, m = _err(lib.irb_gather_region_payload(FAKE, FAKE, 1, 1, 10, 4, FAKE, None, 3, 4, FAKE, FAKE, None))
    assert s == 3 and "16" in m
    s, m = _err(lib.irb_gather_region_payload(ctypes.c_void_p(0x1008), FAKE, 1, 1, 10, 8, FAKE, None, 3, 4, FAKE,
                                              FAKE, None))
    assert s == 3 and "aligned" in m
    assert _err(lib.irb_gather_region_payload(FAKE, FAKE, 1, 1, 10, 8, FAKE, None, 3, 0, FAKE, FAKE, None))[0] == 3
    # summaries need the valid mask
    s, m = _err(lib.irb_summarize_region_payload(FAKE, FAKE, 1, None, 1, 3, 4, 8, FAKE, None))
    assert s == 3 and "NULL" in m
    # selection with the current-region slot: workspace holds the block selection and the region prefix
    lay = _layout(S=64)
    need = lib.irb_select_regions_csa_workspace_size(1, 64, 4, 0)
    assert need >= 64 * 4 * 4
    s, m = _err(lib.irb_select_regions_csa(ctypes.byref(lay), FAKE, 16, 0, 64, None, 4, 4, FAKE, FAKE, FAKE, need - 1,
                                           None))
    assert s == 3 and "workspace" in m
    assert _err(lib.irb_select_regions_csa(ctypes.byref(lay), FAKE, 16, 0, 64, None, 4, 0, FAKE, FAKE, FAKE, need,
                                           None))[0] == 3
    assert _err(lib.irb_select_regions_csa(ctypes.byref(lay), FAKE, 16, 0, 64, None, 4, 4, FAKE, FAKE, FAKE, need,
                                           None))[0] == 1                    # valid; no GPU here
