"""Flat work-item map over ragged sequences (oracle side; test infrastructure only).

Source: the pages credit FlashAttention-2 with parallelising over the
sequence dimension as well as batch and heads, so that long sequences in
small batches still fill the GPU (iplexlaw.co.kr, "FlashAttention-2 GPU work
partitioning", section "Tres mejoras en la utilización de la GPU";
zepes.com, "Comprendiendo Flash-Atención y Flash-Atención-2", section
"FlashAttention-2").  With packed ragged sequences a query block must not
straddle two sequences, so each sequence b is cut into ceil(Lq_b / BM) blocks
of BM query rows.

Definition (reading: canonical order, sequence-major, block-ascending):
    blk_start[0]   = 0
    blk_start[b+1] = blk_start[b] + ceil(Lq_b / BM)
Work item t belongs to the sequence b with blk_start[b] <= t < blk_start[b+1]
and covers query rows [ (t - blk_start[b]) * BM, min(Lq_b, (t - blk_start[b] + 1) * BM) )
of that sequence.
"""
from __future__ import annotations

import numpy as np

from .cu_seqlens import lengths_from_cu


def tile_map(cu_q, block_m: int) -> np.ndarray:
    """Exclusive prefix sum of per-sequence block counts, int32, length batch+1."""
    if block_m <= 0:
        raise ValueError("block_m must be positive")
    lengths = lengths_from_cu(cu_q)
    blk_start = np.zeros(lengths.size + 1, dtype=np.int64)
    for b, L in enumerate(lengths):
        nblk = (int(L) + block_m - 1) // block_m  # ceil(L / BM); 0 for an empty sequence
        blk_start[b + 1] = blk_start[b] + nblk
    if blk_start[-1] > np.iinfo(np.int32).max:
        raise ValueError("too many work items for int32")
    return blk_start.astype(np.int32)


def tile_items(cu_q, block_m: int) -> np.ndarray:
    """The work items (b, m) in map order, int32 [T, 2]."""
    blk_start = tile_map(cu_q, block_m)
    items = []
    for b in range(blk_start.size - 1):
        for m in range(int(blk_start[b + 1] - blk_start[b])):
            items.append((b, m))
    return np.asarray(items, dtype=np.int32).reshape(-1, 2)
