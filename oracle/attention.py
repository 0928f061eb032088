"""Materialised exact attention over packed ragged sequences, float64.

TEST INFRASTRUCTURE (see the package docstring for who may import it).

What is computed -- the plain definition the tiled method reaches exactly up to
floating-point order:
  * Standard attention scores every visible (query, key) pair, normalises the
    scores row by row with a softmax and multiplies the probabilities by the
    values (slavadubrov.com, "O que FlashAttention muda na inferência",
    section "Separar o armazenamento do cálculo").  This function builds that
    score matrix in full, one (sequence, head) at a time.
  * The tiled algorithm keeps attention exact; only the order of
    floating-point operations differs, so results are compared within
    tolerances, not bit for bit (iplexlaw.co.kr, "FlashAttention-2 GPU work
    partitioning", section "Bloques pequeños, normalización global").
  * Sequences are addressed by cumulative offsets; sequence b's query rows are
    cu_q[b] .. cu_q[b+1]-1 of the packed tensor and its key/value rows are
    cu_k[b] .. cu_k[b+1]-1 (friki.work, "Mecanismo cu_seqlens en
    FlashAttention", sections "Estructuras de datos clave" and "Lógica de
    cálculo de longitud").  No query ever sees a key of another sequence.
  * A causal mask may be combined with variable lengths (same page, section
    "Integración con máscaras causales y caché paginada").
  * Several query heads may share one key/value head (multi-query and
    grouped-query attention, zepes.com "Comprendiendo Flash-Atención y
    Flash-Atención-2", section "FlashAttention-2"): with H query heads and Hk
    key/value heads (Hk dividing H), query head h attends with key/value head
    h // (H / Hk).  Hk == H is ordinary multi-head attention.

Readings where the pages are silent:
  * Causal alignment is bottom-right: query i (0-based within its sequence)
    sees key j iff j <= i + Lk - Lq.  With Lq == Lk this is j <= i.
  * A row with no visible key (Lk == 0, or causal with i < Lq - Lk) has
    output 0 and log-sum-exp -inf.
  * lse is the natural log of sum_j exp(scale * q_i . k_j) over visible j,
    stored as [heads, total_q].
  * Inputs are used at the exact values the device receives (bf16 values are
    upcast without change); all arithmetic here is float64.

Layouts: q [Tq, H, D], k and v [Tk, Hk, D]; out [Tq, H, D]; lse [H, Tq].
Rows at or beyond cu_q[-1] belong to no sequence and are returned as NaN.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .cu_seqlens import check_cu_seqlens


def visible_mask(Lq: int, Lk: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), Lk]: True where query i may attend to key j.

    ``rows`` are query indices local to the sequence (default: all Lq rows).
    """
    i = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    if not causal:
        return np.ones((i.size, Lk), dtype=bool)
    j = np.arange(Lk)[None, :]
    return j <= i[:, None] + (Lk - Lq)


def _softmax_rows(S: np.ndarray, vis: np.ndarray, Vb: np.ndarray):
    """Row-wise softmax of S over the visible entries, then times Vb.

    Returns (out [rows, D], lse [rows]).  Rows with no visible entry give a
    zero output and -inf log-sum-exp.
    """
    S = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    mu = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.exp(S - mu[:, None])  # exp(-inf) = 0 for masked entries
    l = E.sum(axis=1)
    out = np.zeros((S.shape[0], Vb.shape[1]), dtype=np.float64)
    lse = np.full(S.shape[0], -np.inf, dtype=np.float64)
    if any_vis.any():
        out[any_vis] = (E[any_vis] @ Vb) / l[any_vis, None]
        lse[any_vis] = mu[any_vis] + np.log(l[any_vis])
    return out, lse


def kv_head_of(H: int, Hk: int) -> int:
    """Query heads per key/value head (the group size); Hk must divide H."""
    if Hk < 1 or H % Hk:
        raise ValueError(f"key/value heads ({Hk}) must divide query heads ({H})")
    return H // Hk


def _check_shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or q.shape[2] != k.shape[2]:
        raise ValueError("expected q [Tq,H,D], k and v [Tk,Hk,D] with equal D")
    return kv_head_of(q.shape[1], k.shape[1])


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, scale: float,
                  causal: bool, heads: Optional[Sequence[int]] = None, row_chunk: int = 1024):
    """Exact varlen attention forward in float64.

    ``heads`` restricts the computation to a subset of query heads (others
    stay NaN).  Rows are processed in chunks of at most ``row_chunk``
    queries, which is still the row-wise definition.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    group = _check_shapes(q, k, v)
    Tq, H, D = q.shape
    Tk = k.shape[0]
    cq = check_cu_seqlens(cu_q, Tq)
    ck = check_cu_seqlens(cu_k, Tk)
    if cq.size != ck.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    hs = range(H) if heads is None else list(heads)
    out = np.full((Tq, H, D), np.nan, dtype=np.float64)
    lse = np.full((H, Tq), np.nan, dtype=np.float64)
    for b in range(cq.size - 1):
        q0, Lq = int(cq[b]), int(cq[b + 1] - cq[b])
        k0, Lk = int(ck[b]), int(ck[b + 1] - ck[b])
        if Lq == 0:
            continue
        for h in hs:
            Kb = k[k0:k0 + Lk, h // group, :].astype(np.float64)
            Vb = v[k0:k0 + Lk, h // group, :].astype(np.float64)
            for r0 in range(0, Lq, row_chunk):
                r1 = min(Lq, r0 + row_chunk)
                Qb = q[q0 + r0:q0 + r1, h, :].astype(np.float64)
                S = scale * (Qb @ Kb.T)
                vis = visible_mask(Lq, Lk, causal, np.arange(r0, r1))
                o, s = _softmax_rows(S, vis, Vb)
                out[q0 + r0:q0 + r1, h, :] = o
                lse[h, q0 + r0:q0 + r1] = s
    return out, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, scale: float,
                   causal: bool, rows: Iterable[int], heads: Iterable[int]):
    """The same definition for selected packed query rows and heads only.

    Returns (out [len(rows), len(heads), D], lse [len(heads), len(rows)]) in
    float64, for sampled checks at sizes where the full oracle is too slow.
    """
    rows = np.asarray(list(rows), dtype=np.int64)
    heads = list(heads)
    group = _check_shapes(q, k, v)
    Tq, H, D = q.shape
    cq = check_cu_seqlens(cu_q, Tq)
    ck = check_cu_seqlens(cu_k, k.shape[0])
    out = np.full((rows.size, len(heads), D), np.nan, dtype=np.float64)
    lse = np.full((len(heads), rows.size), np.nan, dtype=np.float64)
    seq_of = np.searchsorted(cq, rows, side="right") - 1
    for b in np.unique(seq_of):
        b = int(b)
        if b < 0 or b >= cq.size - 1:
            continue  # row outside every sequence: stays NaN
        sel = np.nonzero(seq_of == b)[0]
        q0, Lq = int(cq[b]), int(cq[b + 1] - cq[b])
        k0, Lk = int(ck[b]), int(ck[b + 1] - ck[b])
        local = rows[sel] - q0
        vis = visible_mask(Lq, Lk, causal, local)
        for hi, h in enumerate(heads):
            Kb = k[k0:k0 + Lk, h // group, :].astype(np.float64)
            Vb = v[k0:k0 + Lk, h // group, :].astype(np.float64)
            Qb = q[rows[sel], h, :].astype(np.float64)
            S = scale * (Qb @ Kb.T)
            o, s = _softmax_rows(S, vis, Vb)
            out[sel, hi, :] = o
            lse[hi, sel] = s
    return out, lse


def flops_visible_pairs(cu_q, cu_k, causal: bool) -> int:
    """Number of visible (query, key) pairs, counted from the mask itself."""
    cq = check_cu_seqlens(cu_q)
    ck = check_cu_seqlens(cu_k)
    total = 0
    for b in range(cq.size - 1):
        Lq, Lk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        for r0 in range(0, Lq, 4096):
            r1 = min(Lq, r0 + 4096)
            total += int(visible_mask(Lq, Lk, causal, np.arange(r0, r1)).sum())
    return total
