"""C ABI checks that need no GPU: the library loads, exports every function
that include/fa_varlen.h declares, and host validation returns the documented
status codes before any HIP call is made (so nothing here launches work)."""
import ctypes
import math
import os
import re

import pytest

import variable_length_flashattention_cu_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_varlen.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa_varlen.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["fa_status_string", "fa_varlen_block_sizes", "fa_varlen_tile_map",
                            "fa_varlen_fwd", "fa_varlen_fwd_mapped", "fa_varlen_check_cu_seqlens",
                            "fa_varlen_bwd", "fa_varlen_bwd_workspace_size", "fa_varlen_fwd_kvcache",
                            "fa_varlen_kvcache_workspace_size"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(10):
        s = fa.fa_status_string(code)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(12345) == "unknown status"
    assert fa.fa_status_string(0) == "ok"


def test_block_sizes():
    for d in (64, 96, 128):
        for dt in (fa.FA_DTYPE_F32, fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16):
            bm, bn = fa.fa_varlen_block_sizes(d, dt)
            assert bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
    for dt in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16):
        bm, bn = fa.fa_varlen_block_sizes(256, dt)
        assert bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
    for d, dt in ((80, fa.FA_DTYPE_BF16), (256, fa.FA_DTYPE_F32), (512, fa.FA_DTYPE_BF16)):
        with pytest.raises(fa.FaVarlenError) as e:
            fa.fa_varlen_block_sizes(d, dt)
        assert e.value.status == 4
    with pytest.raises(fa.FaVarlenError) as e:
        fa.fa_varlen_block_sizes(64, 7)
    assert e.value.status == 2
    lib = fa.load_library()
    assert lib.fa_varlen_block_sizes(64, 1, None, None) == 1


# Fake device addresses: validation rejects every call below before any
# pointer is dereferenced or any HIP call is made.
A16 = 0x10000
A4 = 0x10004


def call_fwd(**over):
    args = dict(q=A16, k=A16, v=A16, cu_q=A16, cu_k=A16, max_q=8, max_k=8, scale=0.125, causal=0, out=A16,
                lse=A16, batch=1, total_q=8, total_k=8, heads=2, heads_k=2, head_dim=64, dtype=1)
    args.update(over)
    lib = fa.load_library()
    return lib.fa_varlen_fwd(args["q"], args["k"], args["v"], args["cu_q"], args["cu_k"], args["max_q"],
                             args["max_k"], args["scale"], args["causal"], args["out"], args["lse"],
                             args["batch"], args["total_q"], args["total_k"], args["heads"], args["heads_k"],
                             args["head_dim"], args["dtype"], None)


def call_mapped(**over):
    args = dict(q=A16, k=A16, v=A16, cu_q=A16, cu_k=A16, max_q=8, max_k=8, scale=0.125, causal=0, out=A16,
                lse=A16, batch=1, total_q=8, total_k=8, heads=2, heads_k=2, head_dim=64, dtype=1, blk=A16)
    args.update(over)
    lib = fa.load_library()
    return lib.fa_varlen_fwd_mapped(args["q"], args["k"], args["v"], args["cu_q"], args["cu_k"], args["max_q"],
                                    args["max_k"], args["scale"], args["causal"], args["out"], args["lse"],
                                    args["batch"], args["total_q"], args["total_k"], args["heads"],
                                    args["heads_k"], args["head_dim"], args["dtype"], args["blk"], None)


@pytest.mark.parametrize("call", [call_fwd, call_mapped])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(cu_q=None), 1), (dict(cu_k=None), 1),
    (dict(out=None), 1), (dict(lse=None), 1),
    (dict(dtype=3), 2), (dict(dtype=-1), 2),
    (dict(heads_k=0), 3), (dict(heads_k=3), 3), (dict(heads=4, heads_k=3), 3), (dict(heads_k=-2), 3),
    (dict(head_dim=80), 4), (dict(head_dim=256, dtype=0), 4), (dict(head_dim=512), 4), (dict(head_dim=0), 4),
    (dict(head_dim=32), 4),
    (dict(batch=-1), 3), (dict(total_q=-1), 3), (dict(heads=0), 3), (dict(max_q=9), 3), (dict(max_k=9), 3),
    (dict(max_q=-1), 3),
    (dict(scale=0.0), 6), (dict(scale=-1.0), 6), (dict(scale=math.inf), 6), (dict(scale=math.nan), 6),
    (dict(causal=2), 6), (dict(causal=-1), 6),
    (dict(q=A16 + 8), 5), (dict(k=A16 + 2), 5), (dict(v=A16 + 4), 5), (dict(out=A16 + 8), 5),
    (dict(lse=A16 + 2), 5), (dict(cu_q=A16 + 1), 5), (dict(cu_k=A16 + 2), 5),
])
def test_fwd_validation(call, over, code):
    assert call(**over) == code


def test_shared_kv_heads_dtypes_and_head_dims_pass_validation():
    # valid groupings, dtypes and head dims reach the empty-problem early exit: FA_OK, nothing launched
    for heads, heads_k in ((8, 1), (8, 2), (8, 4), (8, 8), (6, 3)):
        for dtype in (0, 1, 2):
            for head_dim in (64, 96, 128) if dtype == 0 else (64, 96, 128, 256):
                assert call_fwd(heads=heads, heads_k=heads_k, dtype=dtype, head_dim=head_dim, total_q=0,
                                max_q=0) == 0


def test_mapped_needs_map():
    assert call_mapped(blk=None) == 1
    assert call_mapped(blk=A16 + 2) == 5


def test_lse_and_offsets_need_only_4_byte_alignment():
    # with only 4-byte alignment on lse/offsets and an empty batch, nothing is launched: FA_OK
    assert call_fwd(lse=A4, cu_q=A4, cu_k=A4, batch=0, max_q=0, max_k=0) == 0
    assert call_mapped(lse=A4, cu_q=A4, cu_k=A4, batch=0, max_q=0, max_k=0, blk=A4) == 0


def test_empty_problems_launch_nothing():
    assert call_fwd(batch=0, max_q=0, max_k=0) == 0
    assert call_fwd(total_q=0, max_q=0) == 0  # no query rows
    assert call_mapped(total_q=0, max_q=0) == 0


def test_grid_too_large():
    # 2^31-1 rows, one head per ... heads chosen so that work items x heads overflow int32
    big = 2**31 - 1
    assert call_fwd(total_q=big, total_k=8, max_q=big, heads=2**20, head_dim=64) == 8


def test_tile_map_validation():
    lib = fa.load_library()
    assert lib.fa_varlen_tile_map(None, 1, 128, A16, None) == 1
    assert lib.fa_varlen_tile_map(A16, 1, 128, None, None) == 1
    assert lib.fa_varlen_tile_map(A16, -1, 128, A16, None) == 3
    assert lib.fa_varlen_tile_map(A16, 1, 0, A16, None) == 6
    assert lib.fa_varlen_tile_map(A16, 1, 5000, A16, None) == 6
    assert lib.fa_varlen_tile_map(A16 + 1, 1, 128, A16, None) == 5


def test_check_cu_validation():
    lib = fa.load_library()
    assert lib.fa_varlen_check_cu_seqlens(None, A16, 1, 8, 8, 8, 8, A16, None) == 1
    assert lib.fa_varlen_check_cu_seqlens(A16, A16, -1, 8, 8, 8, 8, A16, None) == 3
    assert lib.fa_varlen_check_cu_seqlens(A16, A16, 1, 8, 8, 8, 8, A16 + 2, None) == 5


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "_PKG_DIR", str(tmp_path))
    with pytest.raises(fa.FaVarlenError, match="not built"):
        fa.load_library()
    with pytest.raises(fa.FaVarlenError, match="not built"):
        fa.fa_varlen_block_sizes(64, 1)


# ---------------------------------------------------------------- backward
WS = 1 << 20


def call_bwd(**over):
    args = dict(q=A16, k=A16, v=A16, out=A16, dout=A16, lse=A16, cu_q=A16, cu_k=A16, max_q=8, max_k=8,
                scale=0.125, causal=0, dq=A16, dk=A16, dv=A16, batch=1, total_q=8, total_k=8, heads=2,
                heads_k=2, head_dim=64, dtype=1, ws=A16, ws_bytes=WS)
    args.update(over)
    lib = fa.load_library()
    return lib.fa_varlen_bwd(args["q"], args["k"], args["v"], args["out"], args["dout"], args["lse"],
                             args["cu_q"], args["cu_k"], args["max_q"], args["max_k"], args["scale"],
                             args["causal"], args["dq"], args["dk"], args["dv"], args["batch"], args["total_q"],
                             args["total_k"], args["heads"], args["heads_k"], args["head_dim"], args["dtype"],
                             args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(lse=None), 1), (dict(dout=None), 1), (dict(dq=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1), (dict(cu_k=None), 1),
    (dict(dtype=0), 2), (dict(dtype=3), 2),
    (dict(head_dim=96), 4), (dict(head_dim=256), 4), (dict(head_dim=80), 4),
    (dict(heads_k=3), 3), (dict(max_q=9), 3), (dict(batch=-1), 3),
    (dict(scale=0.0), 6), (dict(causal=2), 6),
    (dict(dout=A16 + 8), 5), (dict(dq=A16 + 2), 5), (dict(dk=A16 + 4), 5), (dict(dv=A16 + 8), 5),
    (dict(ws=A16 + 8), 5),
    (dict(ws=None), 9), (dict(ws_bytes=100), 9), (dict(ws_bytes=0), 9),
])
def test_bwd_validation(over, code):
    assert call_bwd(**over) == code


def test_bwd_workspace_size():
    def size(b, t, h, d):
        n = ctypes.c_size_t(0)
        assert fa.load_library().fa_varlen_bwd_workspace_size(b, t, h, d, ctypes.byref(n)) == 0
        return n.value
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for b, t, h, d in ((1, 8, 2, 64), (2, 300, 2, 64), (23, 65536, 32, 128), (0, 0, 1, 64)):
        assert size(b, t, h, d) == r(t * h * d * 4) + r(h * t * 4) + r((b + 1) * 4)
        assert fa.fa_varlen_bwd_workspace_size(b, t, h, d) == size(b, t, h, d)
    lib = fa.load_library()
    assert lib.fa_varlen_bwd_workspace_size(1, 8, 2, 64, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.fa_varlen_bwd_workspace_size(-1, 8, 2, 64, ctypes.byref(n)) == 3
    assert lib.fa_varlen_bwd_workspace_size(1, 8, 0, 64, ctypes.byref(n)) == 3
    # the exact size passes validation; one byte less does not
    need = size(1, 8, 2, 64)
    assert call_bwd(ws_bytes=need - 1) == 9


# ---------------------------------------------------------------- key/value cache
def call_kv(**over):
    args = dict(q=A16, kc=A16, vc=A16, cu_q=A16, sk=A16, lp=None, bt=None, max_q=1, max_k=8, scale=0.125,
                causal=0, out=A16, lse=A16, batch=1, total_q=1, blocks=1, rows=8, bps=0, heads=2, heads_k=1,
                head_dim=64, dtype=1, splits=0, ws=A16, ws_bytes=1 << 24)
    args.update(over)
    lib = fa.load_library()
    return lib.fa_varlen_fwd_kvcache(args["q"], args["kc"], args["vc"], args["cu_q"], args["sk"], args["lp"],
                                     args["bt"], args["max_q"], args["max_k"], args["scale"], args["causal"],
                                     args["out"], args["lse"], args["batch"], args["total_q"], args["blocks"],
                                     args["rows"], args["bps"], args["heads"], args["heads_k"], args["head_dim"],
                                     args["dtype"], args["splits"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(cu_q=None), 1), (dict(sk=None), 1),
    (dict(out=None), 1), (dict(lse=None), 1),
    (dict(dtype=0), 2), (dict(dtype=5), 2),
    (dict(head_dim=96), 4), (dict(head_dim=256), 4),
    (dict(heads_k=3), 3), (dict(max_q=2), 3), (dict(rows=0), 3), (dict(max_k=9), 3), (dict(blocks=0), 3),
    (dict(bt=A16, bps=0), 3), (dict(bt=A16, bps=1, max_k=9), 3), (dict(batch=-1), 3),
    (dict(scale=0.0), 6), (dict(causal=3), 6), (dict(splits=-1), 6), (dict(splits=65), 6),
    (dict(q=A16 + 8), 5), (dict(kc=A16 + 4), 5), (dict(out=A16 + 2), 5), (dict(lp=A16 + 2), 5),
    (dict(bt=A16 + 1, bps=1), 5), (dict(sk=A16 + 2), 5),
    (dict(ws=None), 9), (dict(ws_bytes=16), 9),
])
def test_kvcache_validation(over, code):
    assert call_kv(**over) == code


def test_kvcache_workspace_size_and_empty():
    lib = fa.load_library()
    n = ctypes.c_size_t(0)
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for t, h, d, s in ((1, 2, 64, 1), (7, 32, 128, 4), (64, 8, 128, 0)):
        assert lib.fa_varlen_kvcache_workspace_size(t, h, d, s, ctypes.byref(n)) == 0
        p = (s if s else 64) * 4
        assert n.value == r(t * h * p * d * 4) + r(t * h * p * 2 * 4)
        assert fa.fa_varlen_kvcache_workspace_size(t, h, d, s) == n.value
    assert lib.fa_varlen_kvcache_workspace_size(1, 2, 64, 65, ctypes.byref(n)) == 6
    assert lib.fa_varlen_kvcache_workspace_size(1, 2, 64, 0, None) == 1
    # no query rows: valid, nothing launched
    assert call_kv(batch=0, total_q=0, max_q=0) == 0
    assert call_kv(total_q=0, max_q=0) == 0
