"""C ABI checks that need no GPU: the library loads, exports every function
that include/fa_varlen.h declares, and host validation of the fa_tensor
descriptors returns the documented status codes before any HIP call is made
(so nothing here launches work: every call below is rejected, or is an empty
problem that returns FA_OK before launching)."""
import ctypes
import math
import os
import re

import pytest

import variable_length_flashattention_cu_amd as fa
from variable_length_flashattention_cu_amd import make_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_varlen.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa_varlen.so not built (run __graft_entry__.build())")

OK, NULL, DTYPE, SHAPE, HEAD_DIM, LAYOUT, ALIGN, ARG, HIP, TOO_LARGE, WORKSPACE, SCRATCH = range(12)
F32, BF16, I32, F16 = fa.FA_DTYPE_F32, fa.FA_DTYPE_BF16, fa.FA_DTYPE_I32, fa.FA_DTYPE_F16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["fa_status_string", "fa_varlen_block_sizes", "fa_varlen_tile_map",
                            "fa_varlen_fwd", "fa_varlen_fwd_mapped", "fa_varlen_fwd_noalloc",
                            "fa_varlen_check_cu_seqlens",
                            "fa_varlen_bwd", "fa_varlen_bwd_workspace_size", "fa_varlen_fwd_kvcache",
                            "fa_varlen_kvcache_workspace_size"])


def test_header_status_and_dtype_values():
    """The status numbering and the descriptor layout are the documented ones."""
    text = open(HEADER).read()
    for name, val in (("FA_OK", 0), ("FA_ERR_NULL", 1), ("FA_ERR_DTYPE", 2), ("FA_ERR_SHAPE", 3),
                      ("FA_ERR_HEAD_DIM", 4), ("FA_ERR_LAYOUT", 5), ("FA_ERR_ALIGN", 6), ("FA_ERR_ARG", 7),
                      ("FA_ERR_HIP", 8), ("FA_DTYPE_F32", 0), ("FA_DTYPE_BF16", 1), ("FA_DTYPE_I32", 2)):
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
    assert ctypes.sizeof(fa.FaTensor) == 8 + 4 + 4 + 3 * 8 + 3 * 8
    assert fa.FaTensor.shape.offset == 16 and fa.FaTensor.stride.offset == 40


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_probe_library_exports_its_header():
    """libfa_probe.so (the measurement aid bench.py uses) exports what include/fa_probe.h declares."""
    path = os.path.join(os.path.dirname(fa.library_path()), "libfa_probe.so")
    if not os.path.exists(path):
        pytest.skip("libfa_probe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))
    assert names == ["fa_probe_mfma_peak", "fa_probe_mfma_peak_random"]
    lib = ctypes.CDLL(path)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(12):
        s = fa.fa_status_string(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert fa.fa_status_string(12345) == "unknown status"
    assert fa.fa_status_string(0) == "ok"


def test_block_sizes():
    for d in (64, 96, 128):
        for dt in (F32, BF16, F16):
            bm, bn = fa.fa_varlen_block_sizes(d, dt)
            assert bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
    for dt in (BF16, F16):
        bm, bn = fa.fa_varlen_block_sizes(256, dt)
        assert bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
    for d, dt in ((80, BF16), (256, F32), (512, BF16)):
        with pytest.raises(fa.FaVarlenError) as e:
            fa.fa_varlen_block_sizes(d, dt)
        assert e.value.status == HEAD_DIM
    for dt in (I32, 7, -1):
        with pytest.raises(fa.FaVarlenError) as e:
            fa.fa_varlen_block_sizes(64, dt)
        assert e.value.status == DTYPE
    lib = fa.load_library()
    assert lib.fa_varlen_block_sizes(64, 1, None, None) == NULL


# Fake device addresses: validation rejects every call below before any
# pointer is dereferenced or any HIP call is made.
A16 = 0x10000


def tensors(**over):
    """Descriptors of a small valid forward problem: batch 1, 8 rows, H=2, Hk=2, D=64, bf16."""
    p = dict(dt=BF16, Tq=8, Tk=8, H=2, Hk=2, D=64, B=1)
    p.update({k: v for k, v in over.items() if k in p})
    t = {"q": make_desc(A16, p["dt"], (p["Tq"], p["H"], p["D"])),
         "k": make_desc(A16, p["dt"], (p["Tk"], p["Hk"], p["D"])),
         "v": make_desc(A16, p["dt"], (p["Tk"], p["Hk"], p["D"])),
         "cu_q": make_desc(A16, I32, (p["B"] + 1,)), "cu_k": make_desc(A16, I32, (p["B"] + 1,)),
         "out": make_desc(A16, p["dt"], (p["Tq"], p["H"], p["D"])),
         "lse": make_desc(A16, F32, (p["H"], p["Tq"])), "blk": make_desc(A16, I32, (p["B"] + 1,))}
    return t


def edit(t, name, **fields):
    d = t[name]
    for f, val in fields.items():
        if f in ("shape", "stride"):
            arr = getattr(d, f)
            for i, x in enumerate(val):
                arr[i] = x
        else:
            setattr(d, f, val)


def call_fwd(t, max_q=8, max_k=8, scale=0.125, causal=0, mapped=False, drop=None, noalloc=False):
    lib = fa.load_library()
    r = {n: (None if n == drop else ctypes.byref(d)) for n, d in t.items()}
    if noalloc:
        return lib.fa_varlen_fwd_noalloc(r["q"], r["k"], r["v"], r["cu_q"], r["cu_k"], max_q, max_k, scale, causal,
                                         r["out"], r["lse"], None)
    if mapped:
        return lib.fa_varlen_fwd_mapped(r["q"], r["k"], r["v"], r["cu_q"], r["cu_k"], max_q, max_k, scale, causal,
                                        r["out"], r["lse"], r["blk"], None)
    return lib.fa_varlen_fwd(r["q"], r["k"], r["v"], r["cu_q"], r["cu_k"], max_q, max_k, scale, causal, r["out"],
                             r["lse"], None)


@pytest.mark.parametrize("mapped", [False, True])
@pytest.mark.parametrize("name", ["q", "k", "v", "cu_q", "cu_k", "out", "lse"])
def test_fwd_null_descriptor(mapped, name):
    assert call_fwd(tensors(), mapped=mapped, drop=name) == NULL


@pytest.mark.parametrize("mapped", [False, True])
@pytest.mark.parametrize("case,code", [
    # element types
    (("q", dict(dtype=I32)), DTYPE), (("q", dict(dtype=9)), DTYPE), (("k", dict(dtype=F16)), DTYPE),
    (("v", dict(dtype=F32)), DTYPE), (("out", dict(dtype=F16)), DTYPE), (("lse", dict(dtype=BF16)), DTYPE),
    (("cu_q", dict(dtype=F32)), DTYPE), (("cu_k", dict(dtype=BF16)), DTYPE),
    # ranks and shapes
    (("q", dict(ndim=2)), SHAPE), (("lse", dict(ndim=3)), SHAPE), (("cu_k", dict(ndim=2)), SHAPE),
    (("q", dict(shape=(-1, 2, 64))), SHAPE), (("k", dict(shape=(8, 3, 64))), SHAPE),
    (("v", dict(shape=(7, 2, 64))), SHAPE), (("out", dict(shape=(8, 2, 128))), SHAPE),
    (("lse", dict(shape=(2, 9))), SHAPE), (("lse", dict(shape=(1, 8))), SHAPE),
    (("cu_k", dict(shape=(3,))), SHAPE), (("cu_q", dict(shape=(0,))), SHAPE),
    (("k", dict(shape=(8, 2, 128))), SHAPE),
    # layout: strides in elements
    (("q", dict(stride=(128, 1, 2))), LAYOUT), (("q", dict(stride=(256, 64, 1))), LAYOUT),
    (("k", dict(stride=(64, 64, 1))), LAYOUT), (("out", dict(stride=(129, 64, 1))), LAYOUT),
    (("lse", dict(stride=(1, 2))), LAYOUT), (("cu_q", dict(stride=(2,))), LAYOUT),
    # data pointers
    (("q", dict(data=None)), NULL), (("lse", dict(data=None)), NULL), (("cu_k", dict(data=None)), NULL),
    # alignment
    (("q", dict(data=A16 + 8)), ALIGN), (("k", dict(data=A16 + 2)), ALIGN), (("v", dict(data=A16 + 4)), ALIGN),
    (("out", dict(data=A16 + 8)), ALIGN), (("lse", dict(data=A16 + 2)), ALIGN),
    (("cu_q", dict(data=A16 + 1)), ALIGN), (("cu_k", dict(data=A16 + 2)), ALIGN),
])
def test_fwd_descriptor_validation(mapped, case, code):
    t = tensors()
    edit(t, case[0], **case[1])
    assert call_fwd(t, mapped=mapped) == code


@pytest.mark.parametrize("mapped", [False, True])
def test_fwd_scalar_validation(mapped):
    t = tensors()
    for kw, code in ((dict(scale=0.0), ARG), (dict(scale=-1.0), ARG), (dict(scale=math.inf), ARG),
                     (dict(scale=math.nan), ARG), (dict(causal=2), ARG), (dict(causal=-1), ARG),
                     (dict(max_q=9), SHAPE), (dict(max_k=9), SHAPE), (dict(max_q=-1), SHAPE)):
        assert call_fwd(t, mapped=mapped, **kw) == code, kw


@pytest.mark.parametrize("mapped", [False, True])
def test_fwd_head_dims_and_groups(mapped):
    for D, dt, code in ((80, BF16, HEAD_DIM), (256, F32, HEAD_DIM), (512, BF16, HEAD_DIM), (32, F16, HEAD_DIM),
                        (0, BF16, HEAD_DIM)):
        assert call_fwd(tensors(D=D, dt=dt), mapped=mapped) == code, (D, dt)
    for H, Hk in ((2, 0), (2, 3), (4, 3), (0, 1)):
        assert call_fwd(tensors(H=H, Hk=Hk), mapped=mapped) == SHAPE, (H, Hk)
    # valid groupings, dtypes and head dims reach the empty-problem early exit: FA_OK, nothing launched
    for H, Hk in ((8, 1), (8, 2), (8, 4), (8, 8), (6, 3)):
        for dt in (F32, BF16, F16):
            for D in (64, 96, 128) if dt == F32 else (64, 96, 128, 256):
                assert call_fwd(tensors(H=H, Hk=Hk, dt=dt, D=D, Tq=0), max_q=0, mapped=mapped) == OK


def test_fwd_layout_of_extent_one_dims_is_free():
    # a dimension of extent 1 may carry any stride (torch gives such views)
    t = tensors(H=1, Hk=1)
    edit(t, "q", stride=(64, 12345, 1))
    edit(t, "lse", stride=(999, 1))
    assert call_fwd(t, max_q=0, max_k=0) == OK  # max_seqlen_q 0: no work item, nothing launched
    t = tensors(H=1, Hk=1, Tq=0)
    edit(t, "q", stride=(64, 12345, 1))
    assert call_fwd(t, max_q=0) == OK


def test_mapped_needs_map():
    t = tensors()
    assert call_fwd(t, mapped=True, drop="blk") == NULL
    edit(t, "blk", data=A16 + 2)
    assert call_fwd(t, mapped=True) == ALIGN
    t = tensors()
    edit(t, "blk", shape=(3,))
    assert call_fwd(t, mapped=True) == SHAPE
    t = tensors()
    edit(t, "blk", dtype=F32)
    assert call_fwd(t, mapped=True) == DTYPE


def test_empty_problems_launch_nothing():
    assert call_fwd(tensors(B=0), max_q=0, max_k=0) == OK
    assert call_fwd(tensors(Tq=0), max_q=0) == OK  # no query rows
    assert call_fwd(tensors(Tq=0), max_q=0, mapped=True) == OK
    # empty tensors may have NULL data
    t = tensors(Tq=0, Tk=0)
    for n in ("q", "k", "v", "out", "lse"):
        edit(t, n, data=None)
    assert call_fwd(t, max_q=0, max_k=0) == OK


def test_noalloc_validation():
    """The no-allocation variant validates like fa_varlen_fwd and refuses
    batches beyond its static map before any HIP call."""
    assert call_fwd(tensors(), noalloc=True, drop="q") == NULL
    t = tensors()
    edit(t, "q", stride=(128, 1, 2))
    assert call_fwd(t, noalloc=True) == LAYOUT
    assert call_fwd(tensors(D=80), noalloc=True) == HEAD_DIM
    assert call_fwd(tensors(), noalloc=True, causal=3) == ARG
    assert call_fwd(tensors(B=65535, Tq=0), max_q=0, noalloc=True) == OK      # largest batch: empty, no launch
    assert call_fwd(tensors(B=65536), noalloc=True) == SCRATCH
    assert call_fwd(tensors(B=65536, Tq=0), max_q=0, noalloc=True) == SCRATCH


def test_grid_too_large():
    big = 2**31 - 1
    assert call_fwd(tensors(Tq=big, H=2**20, Hk=1), max_q=big) == TOO_LARGE
    assert call_fwd(tensors(Tq=2**31), max_q=0) == TOO_LARGE


def test_tile_map_validation():
    lib = fa.load_library()
    cu, blk = make_desc(A16, I32, (2,)), make_desc(A16, I32, (2,))

    def call(cu=cu, blk=blk, max_q=8, d=128, dt=BF16):
        return lib.fa_varlen_tile_map(None if cu is None else ctypes.byref(cu), max_q, d, dt,
                                      None if blk is None else ctypes.byref(blk), None)
    assert call(cu=None) == NULL
    assert call(blk=None) == NULL
    assert call(dt=I32) == DTYPE
    assert call(d=80) == HEAD_DIM
    assert call(max_q=-1) == SHAPE
    assert call(blk=make_desc(A16, I32, (3,))) == SHAPE
    assert call(cu=make_desc(A16, F32, (2,))) == DTYPE
    assert call(cu=make_desc(A16, I32, (2,), (2,))) == LAYOUT
    assert call(cu=make_desc(A16 + 1, I32, (2,))) == ALIGN
    assert call(blk=make_desc(A16 + 2, I32, (2,))) == ALIGN


def test_check_cu_validation():
    lib = fa.load_library()
    cu, flags = make_desc(A16, I32, (2,)), make_desc(A16, I32, (1,))
    b = ctypes.byref
    assert lib.fa_varlen_check_cu_seqlens(None, b(cu), 8, 8, 8, 8, b(flags), None) == NULL
    assert lib.fa_varlen_check_cu_seqlens(b(cu), b(cu), -1, 8, 8, 8, b(flags), None) == SHAPE
    assert lib.fa_varlen_check_cu_seqlens(b(cu), b(make_desc(A16, I32, (3,))), 8, 8, 8, 8, b(flags), None) == SHAPE
    assert lib.fa_varlen_check_cu_seqlens(b(cu), b(cu), 8, 8, 8, 8, b(make_desc(A16 + 2, I32, (1,))), None) == ALIGN


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "_PKG_DIR", str(tmp_path))
    with pytest.raises(fa.FaVarlenError, match="not built"):
        fa.load_library()
    with pytest.raises(fa.FaVarlenError, match="not built"):
        fa.fa_varlen_block_sizes(64, 1)


# ---------------------------------------------------------------- backward
WS = 1 << 20


def bwd_tensors(**over):
    t = tensors(**over)
    t["dout"] = make_desc(A16, t["q"].dtype, list(t["q"].shape))
    t["dq"] = make_desc(A16, t["q"].dtype, list(t["q"].shape))
    t["dk"] = make_desc(A16, t["k"].dtype, list(t["k"].shape))
    t["dv"] = make_desc(A16, t["k"].dtype, list(t["k"].shape))
    return t


def call_bwd(t, max_q=8, max_k=8, scale=0.125, causal=0, ws=A16, ws_bytes=WS, drop=None):
    lib = fa.load_library()
    r = {n: (None if n == drop else ctypes.byref(d)) for n, d in t.items()}
    return lib.fa_varlen_bwd(r["q"], r["k"], r["v"], r["out"], r["dout"], r["lse"], r["cu_q"], r["cu_k"], max_q,
                             max_k, scale, causal, r["dq"], r["dk"], r["dv"], ws, ws_bytes, None)


@pytest.mark.parametrize("name", ["q", "out", "lse", "dout", "dq", "dk", "dv", "cu_k"])
def test_bwd_null_descriptor(name):
    assert call_bwd(bwd_tensors(), drop=name) == NULL


@pytest.mark.parametrize("case,code", [
    (("dout", dict(dtype=F16)), DTYPE), (("dq", dict(dtype=F32)), DTYPE),
    (("dq", dict(shape=(8, 2, 32))), SHAPE), (("dk", dict(shape=(9, 2, 64))), SHAPE),
    (("dv", dict(stride=(128, 1, 2))), LAYOUT), (("dout", dict(stride=(64, 64, 1))), LAYOUT),
    (("dout", dict(data=A16 + 8)), ALIGN), (("dq", dict(data=A16 + 2)), ALIGN), (("dk", dict(data=A16 + 4)), ALIGN),
    (("dv", dict(data=A16 + 8)), ALIGN), (("dq", dict(data=None)), NULL),
])
def test_bwd_descriptor_validation(case, code):
    t = bwd_tensors()
    edit(t, case[0], **case[1])
    assert call_bwd(t) == code


def test_bwd_validation():
    assert call_bwd(bwd_tensors(dt=I32)) == DTYPE
    # head_dim as the forward pass: 256 only for 16-bit inputs
    assert call_bwd(bwd_tensors(dt=F32, D=256)) == HEAD_DIM
    for dt in (BF16, F16, F32):
        for D in (512, 80, 32):
            assert call_bwd(bwd_tensors(D=D, dt=dt)) == HEAD_DIM
    assert call_bwd(bwd_tensors(Hk=3)) == SHAPE
    assert call_bwd(bwd_tensors(), max_q=9) == SHAPE
    assert call_bwd(bwd_tensors(), scale=0.0) == ARG
    assert call_bwd(bwd_tensors(), causal=2) == ARG
    assert call_bwd(bwd_tensors(), ws=A16 + 8) == ALIGN
    assert call_bwd(bwd_tensors(), ws=None) == WORKSPACE
    assert call_bwd(bwd_tensors(), ws_bytes=100) == WORKSPACE
    assert call_bwd(bwd_tensors(), ws_bytes=0) == WORKSPACE


def test_bwd_workspace_size():
    def size(b, t, h, d):
        n = ctypes.c_size_t(0)
        assert fa.load_library().fa_varlen_bwd_workspace_size(b, t, h, d, ctypes.byref(n)) == OK
        return n.value
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for b, t, h, d in ((1, 8, 2, 64), (2, 300, 2, 64), (23, 65536, 32, 128), (0, 0, 1, 64)):
        assert size(b, t, h, d) == r(t * h * d * 4) + r(h * t * 4) + r((b + 1) * 4)
        assert fa.fa_varlen_bwd_workspace_size(b, t, h, d) == size(b, t, h, d)
    lib = fa.load_library()
    assert lib.fa_varlen_bwd_workspace_size(1, 8, 2, 64, None) == NULL
    n = ctypes.c_size_t(0)
    assert lib.fa_varlen_bwd_workspace_size(-1, 8, 2, 64, ctypes.byref(n)) == SHAPE
    assert lib.fa_varlen_bwd_workspace_size(1, 8, 0, 64, ctypes.byref(n)) == SHAPE
    # one byte less than the exact size fails validation
    assert call_bwd(bwd_tensors(), ws_bytes=size(1, 8, 2, 64) - 1) == WORKSPACE


# ---------------------------------------------------------------- key/value cache
def kv_tensors(blocks=1, rows=8, Hk=1, H=2, D=64, B=1, Tq=1, dt=BF16, lp=False, bt=None):
    t = {"q": make_desc(A16, dt, (Tq, H, D)), "kc": make_desc(A16, dt, (blocks * rows, Hk, D)),
         "vc": make_desc(A16, dt, (blocks * rows, Hk, D)), "cu_q": make_desc(A16, I32, (B + 1,)),
         "sk": make_desc(A16, I32, (B,)), "out": make_desc(A16, dt, (Tq, H, D)),
         "lse": make_desc(A16, F32, (H, Tq)), "lp": make_desc(A16, I32, (B,)) if lp else None,
         "bt": make_desc(A16, I32, (B, bt)) if bt else None}
    return t


def call_kv(t, max_q=1, max_k=8, scale=0.125, causal=0, rows=8, splits=0, ws=A16, ws_bytes=1 << 24, drop=None):
    lib = fa.load_library()
    r = {n: (None if (n == drop or d is None) else ctypes.byref(d)) for n, d in t.items()}
    return lib.fa_varlen_fwd_kvcache(r["q"], r["kc"], r["vc"], r["cu_q"], r["sk"], r["lp"], r["bt"], max_q, max_k,
                                     scale, causal, rows, splits, r["out"], r["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("name", ["q", "kc", "vc", "cu_q", "sk", "out", "lse"])
def test_kvcache_null_descriptor(name):
    assert call_kv(kv_tensors(), drop=name) == NULL


def test_kvcache_validation():
    assert call_kv(kv_tensors(dt=I32)) == DTYPE
    for other in (F16, F32):
        t = kv_tensors()
        edit(t, "kc", dtype=other)
        assert call_kv(t) == DTYPE
    t = kv_tensors(dt=F32)
    edit(t, "out", dtype=BF16)
    assert call_kv(t) == DTYPE
    for dt in (BF16, F16, F32):
        for D in (32, 80, 160, 512):
            assert call_kv(kv_tensors(D=D, dt=dt)) == HEAD_DIM
    assert call_kv(kv_tensors(Hk=3)) == SHAPE
    assert call_kv(kv_tensors(), max_q=2) == SHAPE
    assert call_kv(kv_tensors(), rows=0) == SHAPE
    assert call_kv(kv_tensors(), rows=3) == SHAPE            # 8 cache rows are not whole blocks of 3
    assert call_kv(kv_tensors(), max_k=9) == SHAPE
    assert call_kv(kv_tensors(bt=1), max_k=9) == SHAPE
    t = kv_tensors(lp=True)
    edit(t, "lp", shape=(2,))
    assert call_kv(t) == SHAPE
    assert call_kv(kv_tensors(), scale=0.0) == ARG
    assert call_kv(kv_tensors(), causal=3) == ARG
    assert call_kv(kv_tensors(), splits=-1) == ARG
    assert call_kv(kv_tensors(), splits=65) == ARG
    t = kv_tensors()
    edit(t, "kc", stride=(128, 1, 2))
    assert call_kv(t) == LAYOUT
    t = kv_tensors(bt=2)
    edit(t, "bt", stride=(2, 2))  # the last dimension (extent 2) must have stride 1
    assert call_kv(t) == LAYOUT
    for name, off in (("q", 8), ("kc", 4), ("out", 2), ("sk", 2)):
        t = kv_tensors()
        edit(t, name, data=A16 + off)
        assert call_kv(t) == ALIGN, name
    t = kv_tensors(lp=True)
    edit(t, "lp", data=A16 + 2)
    assert call_kv(t) == ALIGN
    t = kv_tensors(bt=1)
    edit(t, "bt", data=A16 + 1)
    assert call_kv(t) == ALIGN
    assert call_kv(kv_tensors(), ws=None) == WORKSPACE
    assert call_kv(kv_tensors(), ws_bytes=16) == WORKSPACE


def test_kvcache_workspace_size_and_empty():
    lib = fa.load_library()
    n = ctypes.c_size_t(0)
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for t, h, d, s in ((1, 2, 64, 1), (7, 32, 128, 4), (64, 8, 128, 0)):
        assert lib.fa_varlen_kvcache_workspace_size(t, h, d, s, ctypes.byref(n)) == OK
        p = s if s else 64
        assert n.value == r(t * h * p * d * 4) + r(t * h * p * 2 * 4)
        assert fa.fa_varlen_kvcache_workspace_size(t, h, d, s) == n.value
    assert lib.fa_varlen_kvcache_workspace_size(1, 2, 64, 65, ctypes.byref(n)) == ARG
    assert lib.fa_varlen_kvcache_workspace_size(1, 2, 64, 0, None) == NULL
    # no query rows: valid, nothing launched
    for dt in (BF16, F16, F32):
        assert call_kv(kv_tensors(B=0, Tq=0, dt=dt), max_q=0) == OK
        assert call_kv(kv_tensors(Tq=0, dt=dt), max_q=0) == OK
