"""Cumulative sequence offsets (oracle side; test infrastructure only).

Source: friki.work, "Mecanismo cu_seqlens en FlashAttention".
  * Section "Estructuras de datos clave": the q and k offset arrays hold
    batch+1 cumulative offsets; [0, 128, 300] describes two sequences of 128
    and 172 tokens.
  * Section "Lógica de cálculo de longitud": the length of sequence b is the
    difference of consecutive entries, offset[b+1] - offset[b], and its
    start is offset[b].
  * Section "Optimización de acceso a memoria": in the variable-length case a
    sequence's first row sits at offset[b] times the row stride (rather than
    b times a fixed batch stride).

Reading where the page is silent: a valid array starts at 0 and never
decreases; its last entry must not exceed the number of packed rows.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def check_cu_seqlens(cu, total_rows: Optional[int] = None) -> np.ndarray:
    """Validate a cumulative-offset array and return it as int64."""
    a = np.asarray(cu)
    if a.ndim != 1 or a.size < 1:
        raise ValueError("cu_seqlens must be a 1-D array of length batch+1")
    if not np.issubdtype(a.dtype, np.integer):
        raise ValueError("cu_seqlens must hold integers")
    a = a.astype(np.int64)
    if a[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if np.any(np.diff(a) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if total_rows is not None and a[-1] > total_rows:
        raise ValueError("cu_seqlens[-1] exceeds the packed row count")
    return a


def lengths_from_cu(cu) -> np.ndarray:
    """Per-sequence lengths: entry b+1 minus entry b."""
    a = check_cu_seqlens(cu)
    return a[1:] - a[:-1]


def row_offset(cu, b: int, row_stride: int) -> int:
    """Element offset of sequence b's first row in a packed [tokens, ...] tensor."""
    a = check_cu_seqlens(cu)
    return int(a[b]) * int(row_stride)
