"""Seeded synthetic inputs for varlen attention.

This module serves both the oracle side (tests, the CPU baseline) and the GPU
side (parity tests, the bench).  It holds no attention arithmetic: only
cumulative-offset construction, Gaussian draws and the bf16 rounding of those
draws, so that both sides receive bit-identical inputs.

Workload shapes follow the FlashAttention pages:
  * cumulative offsets of length batch+1, e.g. [0, 128, 300] for lengths 128
    and 172 (friki.work, "Mecanismo cu_seqlens en FlashAttention",
    section "Estructuras de datos clave");
  * the ragged pair q=[0, 200, 1024] / k=[0, 300, 1024] with 12 heads of
    dimension 64 (same page, section "Ejemplo de uso con PyTorch");
  * sequence lengths 512 to 16k at 16k total tokens per batch, head dimension
    64 and 128, causal and not (iplexlaw.co.kr, "FlashAttention-2 GPU work
    partitioning", section on the roughly 2x kernel speed-up).

Draw recipe: numpy ``default_rng(seed)`` (PCG64); for the ragged 64k batch the
sequence lengths are drawn first; then Q, K and V are drawn in that order as
i.i.d. N(0, 1) float32 arrays of shape [tokens, heads, head_dim] (K and V with
the workload's key/value head count, which may be a divisor of the query head
count: several query heads sharing one key/value head); bf16 and fp16
workloads round each draw to that type with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "bf16_rne_bits",
    "bf16_bits_to_f32",
    "f16_rne_bits",
    "f16_bits_to_f32",
    "cu_from_lengths",
    "loguniform_lengths",
    "workload_tiny",
    "workload_ragged_qk",
    "workload_dense",
    "workload_sweep",
    "workload_ragged64k",
    "workload_custom",
    "workload_ragged64k_gqa",
    "all_parity_workloads",
    "draw_qkv",
    "draw_dout",
    "SWEEP_SEQLENS",
    "SWEEP_HEAD_DIMS",
]

SWEEP_SEQLENS = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP_HEAD_DIMS = (64, 128)


# --------------------------------------------------------------------------
# bf16 rounding of inputs (bit arithmetic; no ml_dtypes in this image)
# --------------------------------------------------------------------------
def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs are finite Gaussian draws, so no
    NaN/Inf handling is needed; finite inputs that overflow become +-inf as
    IEEE rounding prescribes.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE fp16 (round to nearest, ties to even);
    uint16 bit patterns.  numpy's float32 -> float16 cast rounds this way."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of fp16 bit patterns."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# --------------------------------------------------------------------------
# cumulative offsets
# --------------------------------------------------------------------------
def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """int32 cumulative offsets [0, L0, L0+L1, ...] of length batch+1."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if out[-1] > np.iinfo(np.int32).max:
        raise ValueError("total length exceeds int32")
    return out.astype(np.int32)


def loguniform_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> List[int]:
    """Lengths round(exp(U(ln lo, ln hi))) drawn until they reach ``total``.

    The last length is clipped so that the lengths sum to exactly ``total``
    (it may therefore fall below ``lo``).
    """
    lengths: List[int] = []
    acc = 0
    a, b = math.log(lo), math.log(hi)
    while acc < total:
        L = int(round(math.exp(rng.uniform(a, b))))
        L = max(1, min(L, total - acc))
        lengths.append(L)
        acc += L
    return lengths


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cu_q: Tuple[int, ...]
    cu_k: Tuple[int, ...]
    heads: int
    head_dim: int
    dtype: str  # "f32", "bf16" or "f16"
    seed: int
    causal_modes: Tuple[bool, ...]
    lengths_from_rng: bool = False  # ragged 64k: lengths come from the same generator
    heads_k: int = 0  # key/value heads (0: same as heads); must divide heads

    @property
    def kv_heads(self) -> int:
        return self.heads_k or self.heads

    @property
    def batch(self) -> int:
        return len(self.cu_q) - 1

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def lengths_q(self) -> List[int]:
        return [self.cu_q[i + 1] - self.cu_q[i] for i in range(self.batch)]

    @property
    def lengths_k(self) -> List[int]:
        return [self.cu_k[i + 1] - self.cu_k[i] for i in range(self.batch)]

    @property
    def max_seqlen_q(self) -> int:
        return max(self.lengths_q) if self.batch else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.lengths_k) if self.batch else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "batch": self.batch,
            "total_q": self.total_q,
            "total_k": self.total_k,
            "heads": self.heads,
            "kv_heads": self.kv_heads,
            "head_dim": self.head_dim,
            "dtype": self.dtype,
            "seed": self.seed,
        }


def workload_tiny() -> Workload:
    """batch 2, cu=[0,128,300] for q and k, 2 heads, d=64, fp32, non-causal."""
    cu = (0, 128, 300)
    return Workload("tiny_fp32_h2_d64", cu, cu, 2, 64, "f32", 0, (False,))


def workload_ragged_qk() -> Workload:
    """cu_q=[0,200,1024], cu_k=[0,300,1024], 12 heads, d=64, bf16, both masks."""
    return Workload("ragged_qk_h12_d64", (0, 200, 1024), (0, 300, 1024), 12, 64, "bf16", 1,
                    (False, True))


def workload_dense() -> Workload:
    """8 sequences of 2048 tokens, 16 heads, d=128, bf16, both masks."""
    cu = tuple(int(x) for x in cu_from_lengths([2048] * 8))
    return Workload("dense_8x2048_h16_d128", cu, cu, 16, 128, "bf16", 2, (False, True))


def workload_sweep(seqlen: int, head_dim: int) -> Workload:
    """16k total tokens: batch = 16384/seqlen, heads = 2048/head_dim, bf16."""
    if seqlen not in SWEEP_SEQLENS or head_dim not in SWEEP_HEAD_DIMS:
        raise ValueError("sweep point outside the 512..16k x {64,128} grid")
    batch = 16384 // seqlen
    heads = 2048 // head_dim
    idx = SWEEP_SEQLENS.index(seqlen) * len(SWEEP_HEAD_DIMS) + SWEEP_HEAD_DIMS.index(head_dim)
    cu = tuple(int(x) for x in cu_from_lengths([seqlen] * batch))
    return Workload(f"sweep_L{seqlen}_d{head_dim}_h{heads}", cu, cu, heads, head_dim, "bf16",
                    300 + idx, (False, True))


def workload_ragged64k(seed: int = 4, total: int = 65536) -> Workload:
    """64k tokens, lengths log-uniform in [64, 8192], 32 heads, d=128, bf16, causal."""
    rng = np.random.default_rng(seed)
    lengths = loguniform_lengths(rng, total, 64, 8192)
    cu = tuple(int(x) for x in cu_from_lengths(lengths))
    return Workload(f"ragged64k_h32_d128_causal_seed{seed}", cu, cu, 32, 128, "bf16", seed,
                    (True,), lengths_from_rng=True)


def workload_custom(name: str, lengths_q: Sequence[int], lengths_k: Optional[Sequence[int]],
                    heads: int, head_dim: int, dtype: str, seed: int,
                    causal_modes: Tuple[bool, ...] = (False, True), heads_k: int = 0) -> Workload:
    """Any ragged shape (used for edge cases: empty sequences, tails, Lq != Lk),
    optionally with fewer key/value heads than query heads."""
    if heads_k and heads % heads_k:
        raise ValueError("heads_k must divide heads")
    cu_q = tuple(int(x) for x in cu_from_lengths(lengths_q))
    cu_k = cu_q if lengths_k is None else tuple(int(x) for x in cu_from_lengths(lengths_k))
    return Workload(name, cu_q, cu_k, heads, head_dim, dtype, seed, causal_modes, heads_k=heads_k)


def workload_ragged64k_gqa(seed: int = 4, total: int = 65536, heads_k: int = 8) -> Workload:
    """The ragged 64k batch with 32 query heads sharing ``heads_k`` key/value heads."""
    base = workload_ragged64k(seed, total)
    return dataclasses.replace(base, name=f"ragged64k_h32_kv{heads_k}_d128_causal_seed{seed}", heads_k=heads_k)


def draw_dout(wl: Workload) -> dict:
    """Output gradient for the backward pass: standard normal [total_q, heads,
    head_dim] from its own stream (seed + 7919, so Q, K and V are unchanged),
    rounded to the workload's type like the inputs.  Returns ``dout`` (float32)
    and, for 16-bit types, ``dout_bits``."""
    rng = np.random.default_rng(wl.seed + 7919)
    shape = (wl.total_q, wl.heads, wl.head_dim)
    x = rng.standard_normal(shape, dtype=np.float32)
    rounders = {"bf16": (bf16_rne_bits, bf16_bits_to_f32), "f16": (f16_rne_bits, f16_bits_to_f32)}
    if wl.dtype in rounders:
        to_bits, to_f32 = rounders[wl.dtype]
        bits = to_bits(x).reshape(shape)
        return {"dout": to_f32(bits).reshape(shape), "dout_bits": bits}
    if wl.dtype != "f32":
        raise ValueError(wl.dtype)
    return {"dout": x}


def all_parity_workloads() -> List[Workload]:
    out = [workload_tiny(), workload_ragged_qk(), workload_dense()]
    out += [workload_sweep(L, d) for L in SWEEP_SEQLENS for d in SWEEP_HEAD_DIMS]
    out.append(workload_ragged64k())
    return out


def draw_qkv(wl: Workload, heads: Optional[Sequence[int]] = None) -> dict:
    """Draw Q, K, V for a workload.

    Returns float32 arrays ``q``, ``k``, ``v`` (values exactly representable
    in bf16 when the workload is bf16) and, for bf16, the uint16 bit arrays
    ``q_bits``, ``k_bits``, ``v_bits`` that are handed to the device.
    ``heads`` optionally keeps a subset of query heads (the full tensors are
    still drawn so that the values do not depend on the subset); K and V are
    always returned whole.
    """
    rng = np.random.default_rng(wl.seed)
    if wl.lengths_from_rng:
        lengths = loguniform_lengths(rng, wl.total_q, 64, 8192)
        if tuple(cu_from_lengths(lengths)) != tuple(wl.cu_q):
            raise RuntimeError("length draw does not reproduce the workload")
    shape_q = (wl.total_q, wl.heads, wl.head_dim)
    shape_k = (wl.total_k, wl.kv_heads, wl.head_dim)
    rounders = {"bf16": (bf16_rne_bits, bf16_bits_to_f32), "f16": (f16_rne_bits, f16_bits_to_f32)}
    out = {}
    for name, shape in (("q", shape_q), ("k", shape_k), ("v", shape_k)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if wl.dtype in rounders:
            to_bits, to_f32 = rounders[wl.dtype]
            bits = to_bits(x)
            del x
            x = to_f32(bits).reshape(shape)
            bits = bits.reshape(shape)
            if heads is not None and name == "q":
                bits = np.ascontiguousarray(bits[:, list(heads), :])
            out[name + "_bits"] = bits
        elif wl.dtype != "f32":
            raise ValueError(wl.dtype)
        if heads is not None and name == "q":
            x = np.ascontiguousarray(x[:, list(heads), :])
        out[name] = x
    return out


# ---------------------------------------------------------------------------
# key/value-cache (decode-shaped) workloads
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class KVWorkload:
    """Packed queries against a key/value cache.

    Sequence b has ``lengths_q[b]`` query rows and uses cache positions
    ``leftpad[b] .. seqlens_k[b]-1``.  Without paging each sequence owns one
    slot of ``cache_rows`` rows; with paging the cache holds blocks of
    ``cache_rows`` rows and a block table maps a sequence's pages to shuffled
    blocks.  Unused cache rows hold random values too."""
    name: str
    lengths_q: Tuple[int, ...]
    seqlens_k: Tuple[int, ...]
    leftpad: Optional[Tuple[int, ...]]
    heads: int
    kv_heads: int
    head_dim: int
    dtype: str
    seed: int
    cache_rows: int
    paged: bool = False

    @property
    def batch(self) -> int:
        return len(self.lengths_q)

    @property
    def cu_q(self) -> Tuple[int, ...]:
        return tuple(int(x) for x in cu_from_lengths(self.lengths_q))

    @property
    def total_q(self) -> int:
        return int(sum(self.lengths_q))

    @property
    def max_seqlen_q(self) -> int:
        return max(self.lengths_q) if self.lengths_q else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.seqlens_k) if self.seqlens_k else 0

    @property
    def key_lengths(self) -> List[int]:
        lp = self.leftpad or (0,) * self.batch
        return [s - p for s, p in zip(self.seqlens_k, lp)]

    @property
    def blocks_per_seq(self) -> int:
        return max(1, -(-self.max_seqlen_k // self.cache_rows)) if self.paged else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def draw_kvcache(wl: KVWorkload) -> dict:
    """q, k_cache, v_cache as float32 values (exactly representable in the
    workload's type) with, for bf16 and f16, the 16-bit bit arrays ``*_bits``
    handed to the device, and, for a paged cache, the int32 block table
    [batch, blocks_per_seq] (unused entries 0)."""
    rng = np.random.default_rng(wl.seed)
    rounders = {"bf16": (bf16_rne_bits, bf16_bits_to_f32), "f16": (f16_rne_bits, f16_bits_to_f32)}
    if wl.dtype not in rounders and wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype}")
    out = {}
    if wl.paged:
        need = [-(-s // wl.cache_rows) for s in wl.seqlens_k]
        nblk = sum(need) + 3
        order = rng.permutation(nblk)
        table = np.zeros((wl.batch, wl.blocks_per_seq), dtype=np.int32)
        n = 0
        for b, k in enumerate(need):
            table[b, :k] = order[n:n + k]
            n += k
        out["block_table"] = table
        cache_shape = (nblk, wl.cache_rows, wl.kv_heads, wl.head_dim)
    else:
        cache_shape = (wl.batch, wl.cache_rows, wl.kv_heads, wl.head_dim)
    for name, shape in (("q", (wl.total_q, wl.heads, wl.head_dim)), ("k_cache", cache_shape),
                        ("v_cache", cache_shape)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if wl.dtype in rounders:
            to_bits, to_f32 = rounders[wl.dtype]
            bits = to_bits(x).reshape(shape)
            out[name + "_bits"] = bits
            x = to_f32(bits).reshape(shape)
        out[name] = x
    return out


def workload_decode(name: str, lengths_q, seqlens_k, heads: int, kv_heads: int, head_dim: int, dtype: str,
                    seed: int, cache_rows: int, leftpad=None, paged: bool = False) -> KVWorkload:
    if heads % kv_heads:
        raise ValueError("kv_heads must divide heads")
    if leftpad is not None and any(p > s for p, s in zip(leftpad, seqlens_k)):
        raise ValueError("leftpad must not exceed seqlens_k")
    if not paged and max(seqlens_k, default=0) > cache_rows:
        raise ValueError("a sequence longer than its cache slot")
    return KVWorkload(name, tuple(int(x) for x in lengths_q), tuple(int(x) for x in seqlens_k),
                      None if leftpad is None else tuple(int(x) for x in leftpad), heads, kv_heads, head_dim,
                      dtype, seed, cache_rows, paged)


def workload_decode_bench(seed: int = 9) -> KVWorkload:
    """Single-token decoding: 32 sequences with cached lengths log-uniform in
    [1024, 16384], 32 query heads on 8 key/value heads, d=128, bf16, a paged
    cache of 256-row blocks."""
    rng = np.random.default_rng(seed)
    seqlens = [int(round(math.exp(rng.uniform(math.log(1024), math.log(16384))))) for _ in range(32)]
    return workload_decode(f"decode_b32_h32_kv8_d128_paged256_seed{seed}", [1] * 32, seqlens, 32, 8, 128, "bf16",
                           seed, 256, paged=True)
