"""Attention against a key/value cache (the decode-shaped case), float64.

TEST INFRASTRUCTURE (see the package docstring for who may import it).

What is computed: the same exact attention as :mod:`oracle.attention`, with
each sequence's keys and values taken from a cache instead of a packed
tensor:

  * The per-sequence key length need not be given cumulatively: a plain
    array of lengths is one of the two formats, and a left padding may be
    subtracted from it (friki.work, "Mecanismo cu_seqlens en
    FlashAttention", sections "Lógica de cálculo de longitud" and
    "Optimización de acceso a memoria": with the non-cumulative format the
    sequence's keys are addressed by its batch index times a batch stride,
    and the usable key length is the given length minus the left padding).
  * The cache may be paged (same page, section "Integración con máscaras
    causales y caché paginada", which names the paged key/value cache but
    prints no layout).
  * Prefill and token-by-token decoding are different workloads whose
    available parallelism differs, and the cache layout is part of what an
    implementation must support (slavadubrov.com, "O que FlashAttention muda
    na inferência", section "A implementação e a carga de trabalho continuam
    a importar"; iplexlaw.co.kr, "FlashAttention-2 GPU work partitioning",
    section "Cómo documentar una diferencia técnica"): decoding has few query
    rows per sequence.

Readings where the pages are silent:
  * Non-paged cache: ``k_cache[b, p]`` holds position p of sequence b
    (``[batch, cache_rows, Hk, D]``).  Sequence b's keys are positions
    ``leftpad_k[b] .. seqlens_k[b]-1``; its key length is
    ``seqlens_k[b] - leftpad_k[b]`` (leftpad 0 when not given).
  * Paged cache: ``k_cache[blk, r]`` (``[num_blocks, page_size, Hk, D]``);
    position p of sequence b lives in block ``block_table[b, p // page_size]``,
    row ``p % page_size``.
  * Queries are packed by cumulative offsets ``cu_seqlens_q`` as in the
    forward pass; the causal mask is bottom-right over (Lq_b, Lk_b), so a
    single new query token sees every cached key.

The keys and values of each sequence are gathered into packed tensors with
cumulative offsets, and :func:`oracle.attention.attention_fwd` -- the pinned
definition -- does the rest.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import attention_fwd
from .cu_seqlens import check_cu_seqlens


def cache_positions(batch: int, seqlens_k, leftpad_k=None):
    """Per sequence, the cache positions that hold its keys (leftpad .. seqlen-1)."""
    seqlens_k = np.asarray(seqlens_k, dtype=np.int64)
    if seqlens_k.shape != (batch,):
        raise ValueError("seqlens_k must have one entry per sequence")
    lp = np.zeros(batch, dtype=np.int64) if leftpad_k is None else np.asarray(leftpad_k, dtype=np.int64)
    if lp.shape != (batch,) or (lp < 0).any() or (lp > seqlens_k).any():
        raise ValueError("leftpad_k must satisfy 0 <= leftpad_k <= seqlens_k")
    return [np.arange(lp[b], seqlens_k[b]) for b in range(batch)]


def gather_cache(cache: np.ndarray, positions, block_table: Optional[np.ndarray] = None,
                 page_size: Optional[int] = None) -> np.ndarray:
    """Rows of each sequence, in position order, packed back to back: [sum L, Hk, D]."""
    rows = []
    for b, pos in enumerate(positions):
        if block_table is None:
            if pos.size and pos[-1] >= cache.shape[1]:
                raise ValueError("sequence longer than its cache slot")
            rows.append(cache[b, pos])
        else:
            blk = np.asarray(block_table)[b, pos // page_size]
            rows.append(cache[blk, pos % page_size])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.concatenate(rows, axis=0)


def attention_kvcache(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, cu_q, seqlens_k,
                      scale: float, causal: bool, leftpad_k=None, block_table=None, page_size=None):
    """Exact attention of packed queries against a (paged) key/value cache.

    Returns (out [Tq, H, D], lse [H, Tq]) in float64, as attention_fwd.
    """
    cq = check_cu_seqlens(cu_q, q.shape[0])
    batch = cq.size - 1
    if block_table is not None and (page_size is None or page_size != k_cache.shape[1]):
        raise ValueError("a paged cache needs page_size equal to its rows per block")
    pos = cache_positions(batch, seqlens_k, leftpad_k)
    k = gather_cache(np.asarray(k_cache), pos, block_table, page_size)
    v = gather_cache(np.asarray(v_cache), pos, block_table, page_size)
    cu_k = np.concatenate([[0], np.cumsum([p.size for p in pos])]).astype(np.int64)
    return attention_fwd(q, k, v, cq, cu_k, scale, causal)
