"""Python binding of libfa_varlen.so (exact varlen attention, forward and
backward, MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/fa_varlen.h``.  PyTorch supplies device
memory and the stream; no CPU fallback exists -- when the library is not
built every entry point raises :class:`FaVarlenError`.

Functions carry the names of the C entry points:
  fa_varlen_fwd, fa_varlen_fwd_mapped, fa_varlen_fwd_noalloc, fa_varlen_bwd,
  fa_varlen_bwd_workspace_size, fa_varlen_fwd_kvcache,
  fa_varlen_kvcache_workspace_size, fa_varlen_tile_map, fa_varlen_block_sizes,
  fa_varlen_check_cu_seqlens, fa_status_string.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FaVarlenError",
    "FA_DTYPE_F32",
    "FA_DTYPE_BF16",
    "FA_DTYPE_F16",
    "FA_DTYPE_I32",
    "FaTensor",
    "make_desc",
    "desc",
    "library_path",
    "load_library",
    "fa_status_string",
    "fa_varlen_block_sizes",
    "fa_varlen_tile_map",
    "fa_varlen_fwd",
    "fa_varlen_fwd_mapped",
    "fa_varlen_fwd_noalloc",
    "fa_varlen_bwd",
    "fa_varlen_bwd_workspace_size",
    "fa_varlen_fwd_kvcache",
    "fa_varlen_kvcache_workspace_size",
    "fa_varlen_check_cu_seqlens",
]

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_I32 = 2
FA_DTYPE_F16 = 3

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_DTYPE", 3: "FA_ERR_SHAPE", 4: "FA_ERR_HEAD_DIM",
    5: "FA_ERR_LAYOUT", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ARG", 8: "FA_ERR_HIP", 9: "FA_ERR_TOO_LARGE",
    10: "FA_ERR_WORKSPACE", 11: "FA_ERR_SCRATCH",
}

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaVarlenError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({_status_text(status)})")


class FaTensor(ctypes.Structure):
    """The fa_tensor descriptor of include/fa_varlen.h (element strides)."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


def make_desc(data: int, dtype: int, shape, stride=None) -> FaTensor:
    """Descriptor from raw values; stride defaults to row-major contiguous."""
    shape = [int(x) for x in shape]
    if stride is None:
        stride, acc = [0] * len(shape), 1
        for i in range(len(shape) - 1, -1, -1):
            stride[i] = acc
            acc *= shape[i]
    d = FaTensor()
    d.data = int(data) if data else None
    d.dtype = int(dtype)
    d.ndim = len(shape)
    for i, (n, st) in enumerate(zip(shape, stride)):
        d.shape[i] = n
        d.stride[i] = int(st)
    return d


def library_path() -> str:
    return os.path.join(_PKG_DIR, "libfa_varlen.so")


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise FaVarlenError(-1, f"HIP library not built: {path} is missing; run "
                                "`python -m variable_length_flashattention_cu_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    i32p, szp = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)
    tp = ctypes.POINTER(FaTensor)
    sigs = {
        "fa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "fa_varlen_block_sizes": ([i32, i32, i32p, i32p], ctypes.c_int),
        "fa_varlen_tile_map": ([tp, i32, i32, i32, tp, vp], ctypes.c_int),
        "fa_varlen_fwd": ([tp, tp, tp, tp, tp, i32, i32, f32, i32, tp, tp, vp], ctypes.c_int),
        "fa_varlen_fwd_mapped": ([tp, tp, tp, tp, tp, i32, i32, f32, i32, tp, tp, tp, vp], ctypes.c_int),
        "fa_varlen_fwd_noalloc": ([tp, tp, tp, tp, tp, i32, i32, f32, i32, tp, tp, vp], ctypes.c_int),
        "fa_varlen_bwd": ([tp, tp, tp, tp, tp, tp, tp, tp, i32, i32, f32, i32, tp, tp, tp, vp, sz, vp],
                          ctypes.c_int),
        "fa_varlen_bwd_workspace_size": ([i32, i32, i32, i32, szp], ctypes.c_int),
        "fa_varlen_fwd_kvcache": ([tp, tp, tp, tp, tp, tp, tp, i32, i32, f32, i32, i32, i32, tp, tp, vp, sz, vp],
                                  ctypes.c_int),
        "fa_varlen_kvcache_workspace_size": ([i32, i32, i32, i32, szp], ctypes.c_int),
        "fa_varlen_check_cu_seqlens": ([tp, tp, i32, i32, i32, i32, tp, vp], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().fa_status_string(int(status)).decode()
    except Exception:  # library missing: the message names the problem already
        return "library unavailable"


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaVarlenError(status, where)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_varlen_block_sizes(head_dim: int, dtype: int) -> Tuple[int, int]:
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().fa_varlen_block_sizes(int(head_dim), int(dtype), ctypes.byref(bm), ctypes.byref(bn)),
           "fa_varlen_block_sizes")
    return bm.value, bn.value


# --------------------------------------------------------------------------
# torch-facing helpers (torch is only used for memory and streams)
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16, torch.int32: FA_DTYPE_I32,
             torch.float16: FA_DTYPE_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, float16 or int32)")
    return codes[t.dtype]


def desc(t) -> FaTensor:
    """fa_tensor descriptor of a torch tensor (1 to 3 dimensions), or None for None."""
    if t is None:
        return None
    if not 1 <= t.dim() <= 3:
        raise ValueError(f"fa_tensor holds 1 to 3 dimensions, got {t.dim()}")
    return make_desc(t.data_ptr(), _dtype_code(t), t.shape, t.stride())


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_i32(t, name: str):
    torch = _torch()
    if not (t.is_cuda and t.dtype == torch.int32 and t.dim() == 1 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous int32 CUDA tensor of shape [batch+1]")
    return t


def fa_varlen_tile_map(cu_seqlens_q, max_seqlen_q: int, head_dim: int, dtype: int, blk_start=None, stream=None):
    """int32 [batch+1] work-item map of the ragged batch for (head_dim, dtype) (device tensor)."""
    torch = _torch()
    cu = _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    batch = cu.numel() - 1
    if blk_start is None:
        blk_start = torch.empty(batch + 1, dtype=torch.int32, device=cu.device)
    _dev_i32(blk_start, "blk_start")
    d_cu, d_blk = desc(cu), desc(blk_start)
    _check(load_library().fa_varlen_tile_map(ctypes.byref(d_cu), int(max_seqlen_q), int(head_dim), int(dtype),
                                             ctypes.byref(d_blk), _stream_handle(stream)), "fa_varlen_tile_map")
    return blk_start


def _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse):
    torch = _torch()
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[2] != k.shape[2]:
        raise ValueError("expected q [total_q, H, D], k and v [total_k, Hk, D]")
    if k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise ValueError("the key/value head count must divide the query head count")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must be CUDA tensors of one dtype")
    _dtype_code(q)
    cu_q = _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _dev_i32(cu_seqlens_k, "cu_seqlens_k")
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    total_q, H, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous CUDA tensor shaped and typed like q")
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 CUDA tensor of shape [H, total_q]")
    return q, k, v, cu_q, cu_k, float(softmax_scale), out, lse


def fa_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                  softmax_scale: Optional[float] = None, causal: bool = False, out=None, lse=None,
                  stream=None):
    """Exact attention forward over packed variable-length sequences.

    q [total_q, H, D], k/v [total_k, Hk, D] (bf16, fp16 or fp32, CUDA; Hk
    divides H, query head h uses key/value head h // (H // Hk));
    cu_seqlens_* int32 [batch+1] on the device.  Returns (out, lse) with
    out shaped like q and lse float32 [H, total_q].
    """
    q, k, v, cu_q, cu_k, scale, out, lse = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse)
    ds = [desc(x) for x in (q, k, v, cu_q, cu_k, out, lse)]
    st = load_library().fa_varlen_fwd(*map(ctypes.byref, ds[:5]), int(max_seqlen_q), int(max_seqlen_k), scale,
                                      int(bool(causal)), ctypes.byref(ds[5]), ctypes.byref(ds[6]),
                                      _stream_handle(stream))
    _check(st, "fa_varlen_fwd")
    return out, lse


def fa_varlen_fwd_mapped(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                         blk_start, softmax_scale: Optional[float] = None, causal: bool = False, out=None,
                         lse=None, stream=None):
    """fa_varlen_fwd with a work-item map built by fa_varlen_tile_map."""
    q, k, v, cu_q, cu_k, scale, out, lse = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse)
    _dev_i32(blk_start, "blk_start")
    ds = [desc(x) for x in (q, k, v, cu_q, cu_k, out, lse, blk_start)]
    st = load_library().fa_varlen_fwd_mapped(*map(ctypes.byref, ds[:5]), int(max_seqlen_q), int(max_seqlen_k),
                                             scale, int(bool(causal)), ctypes.byref(ds[5]), ctypes.byref(ds[6]),
                                             ctypes.byref(ds[7]), _stream_handle(stream))
    _check(st, "fa_varlen_fwd_mapped")
    return out, lse


def fa_varlen_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, out, lse,
                          softmax_scale: Optional[float] = None, causal: bool = False, stream=None):
    """fa_varlen_fwd that allocates nothing: the caller passes out and lse,
    and the library keeps the work-item map in its static per-GPU array (at
    most 65535 sequences; overlapping calls on one GPU race on it)."""
    if out is None or lse is None:
        raise ValueError("fa_varlen_fwd_noalloc needs caller-allocated out and lse")
    q, k, v, cu_q, cu_k, scale, out, lse = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse)
    ds = [desc(x) for x in (q, k, v, cu_q, cu_k, out, lse)]
    st = load_library().fa_varlen_fwd_noalloc(*map(ctypes.byref, ds[:5]), int(max_seqlen_q), int(max_seqlen_k),
                                              scale, int(bool(causal)), ctypes.byref(ds[5]), ctypes.byref(ds[6]),
                                              _stream_handle(stream))
    _check(st, "fa_varlen_fwd_noalloc")
    return out, lse


def fa_varlen_bwd_workspace_size(batch: int, total_q: int, num_heads: int, head_dim: int) -> int:
    """Bytes of device workspace fa_varlen_bwd needs."""
    n = ctypes.c_size_t(0)
    _check(load_library().fa_varlen_bwd_workspace_size(int(batch), int(total_q), int(num_heads), int(head_dim),
                                                       ctypes.byref(n)), "fa_varlen_bwd_workspace_size")
    return n.value


def _workspace(workspace, need: int, device):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not workspace.is_cuda:
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    return workspace


def fa_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                  softmax_scale: Optional[float] = None, causal: bool = False, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Gradients (dq, dk, dv) of fa_varlen_fwd given dout, the forward's out and lse.

    bf16 or fp16 inputs at head_dim 64, 96, 128 or 256, fp32 at 64, 96 or 128
    (the forward pass's set).  dq is shaped like q, dk and dv
    like k.  ``workspace`` (a CUDA byte tensor of at least
    fa_varlen_bwd_workspace_size bytes) is allocated when not given.
    """
    torch = _torch()
    q, k, v, cu_q, cu_k, scale, out, lse = _prepare(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse)
    dout = dout.contiguous()
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_cuda:
        raise ValueError("dout must be a CUDA tensor shaped and typed like q")
    total_q, H, D = q.shape
    batch = cu_q.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous CUDA tensor shaped and typed like its input")
    workspace = _workspace(workspace, fa_varlen_bwd_workspace_size(batch, total_q, H, D), q.device)
    ds = [desc(x) for x in (q, k, v, out, dout, lse, cu_q, cu_k, dq, dk, dv)]
    st = load_library().fa_varlen_bwd(*map(ctypes.byref, ds[:8]), int(max_seqlen_q), int(max_seqlen_k), scale,
                                      int(bool(causal)), *map(ctypes.byref, ds[8:]), workspace.data_ptr(),
                                      workspace.numel(), _stream_handle(stream))
    _check(st, "fa_varlen_bwd")
    return dq, dk, dv


def fa_varlen_kvcache_workspace_size(total_q: int, num_heads: int, head_dim: int, num_splits: int = 0) -> int:
    """Bytes of device workspace fa_varlen_fwd_kvcache needs."""
    n = ctypes.c_size_t(0)
    _check(load_library().fa_varlen_kvcache_workspace_size(int(total_q), int(num_heads), int(head_dim),
                                                           int(num_splits), ctypes.byref(n)),
           "fa_varlen_kvcache_workspace_size")
    return n.value


def fa_varlen_fwd_kvcache(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                          softmax_scale: Optional[float] = None, causal: bool = False, leftpad_k=None,
                          block_table=None, num_splits: int = 0, out=None, lse=None, workspace=None, stream=None):
    """Attention of packed queries against a key/value cache.

    q [total_q, H, D] (bf16/fp16/fp32, CUDA; D 64, 96, 128 or 256) packed by cu_seqlens_q; k_cache,
    v_cache [blocks, rows, Hk, D]; seqlens_k int32 [batch] (not cumulative);
    optional leftpad_k int32 [batch] and block_table int32 [batch, blocks_per_seq]
    (without one, block b is sequence b's slot).  Returns (out, lse).
    """
    torch = _torch()
    q = q.contiguous()
    k_cache, v_cache = k_cache.contiguous(), v_cache.contiguous()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape or q.shape[2] != k_cache.shape[3]:
        raise ValueError("expected q [total_q, H, D] and caches [blocks, rows, Hk, D]")
    if k_cache.shape[2] < 1 or q.shape[1] % k_cache.shape[2]:
        raise ValueError("the key/value head count must divide the query head count")
    if q.dtype != k_cache.dtype or q.dtype != v_cache.dtype or not (q.is_cuda and k_cache.is_cuda):
        raise TypeError("q and the caches must be CUDA tensors of one dtype")
    _dtype_code(q)
    cu_q = _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    batch = cu_q.numel() - 1
    sk = _dev_i32(seqlens_k, "seqlens_k")
    if sk.numel() != batch:
        raise ValueError("seqlens_k must have one entry per sequence")
    lp = None
    if leftpad_k is not None:
        lp = _dev_i32(leftpad_k, "leftpad_k")
        if lp.numel() != batch:
            raise ValueError("leftpad_k must have one entry per sequence")
    if block_table is not None:
        if not (block_table.is_cuda and block_table.dtype == torch.int32 and block_table.dim() == 2
                and block_table.shape[0] == batch and block_table.is_contiguous()):
            raise TypeError("block_table must be a contiguous int32 CUDA tensor [batch, blocks_per_seq]")
    total_q, H, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous CUDA tensor shaped and typed like q")
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 CUDA tensor of shape [H, total_q]")
    workspace = _workspace(workspace, fa_varlen_kvcache_workspace_size(total_q, H, D, num_splits), q.device)
    blocks, rows, Hk = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    # the caches go over the ABI with their block and row dimensions merged
    kc, vc = k_cache.view(blocks * rows, Hk, D), v_cache.view(blocks * rows, Hk, D)
    ds = [desc(x) for x in (q, kc, vc, cu_q, sk, lp, block_table, out, lse)]
    st = load_library().fa_varlen_fwd_kvcache(
        *map(_ref, ds[:7]), int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale), int(bool(causal)),
        int(rows), int(num_splits), _ref(ds[7]), _ref(ds[8]), workspace.data_ptr(), workspace.numel(),
        _stream_handle(stream))
    _check(st, "fa_varlen_fwd_kvcache")
    return out, lse


def fa_varlen_check_cu_seqlens(cu_seqlens_q, cu_seqlens_k, total_q: int, total_k: int, max_seqlen_q: int,
                               max_seqlen_k: int, flags=None, stream=None):
    """Device check of the offset preconditions; returns an int32 [1] flag tensor."""
    torch = _torch()
    cu_q = _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _dev_i32(cu_seqlens_k, "cu_seqlens_k")
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=cu_q.device)
    d = [desc(x) for x in (cu_q, cu_k, flags)]
    _check(load_library().fa_varlen_check_cu_seqlens(
        ctypes.byref(d[0]), ctypes.byref(d[1]), int(total_q), int(total_k), int(max_seqlen_q), int(max_seqlen_k),
        ctypes.byref(d[2]), _stream_handle(stream)), "fa_varlen_check_cu_seqlens")
    return flags
