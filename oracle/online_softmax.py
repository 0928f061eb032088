"""Tile-by-tile online softmax in float64 (oracle side; test infrastructure only).

Source: the first FlashAttention already split the data into blocks processed
in fast on-chip memory; its online softmax updates and rescales running
statistics and partial outputs so that the normalisation stays global, and
normalising each block on its own and adding the results is *not* the same
computation (iplexlaw.co.kr, "FlashAttention-2 GPU work partitioning",
section "Bloques pequeños, normalización global").  The method keeps
normalisation statistics and output accumulators up to date during the
computation instead of writing all probabilities to HBM (slavadubrov.com,
"O que FlashAttention muda na inferência", section "Separar o armazenamento do
cálculo").

These functions exist only so that tests can pin that equivalence claim:
``online_softmax_attention`` must equal :func:`oracle.attention.attention_fwd`
to float64 rounding, and ``blockwise_normalised_attention`` (normalise every
key block separately, then add) must not.  Neither is used to check the GPU.

Running statistics for one query row, key blocks n = 0, 1, ...:
    m_n   = max(m_{n-1}, max_j s_j)               (row maximum so far)
    alpha = exp(m_{n-1} - m_n)                    (rescale of earlier blocks)
    l_n   = alpha * l_{n-1} + sum_j exp(s_j - m_n)
    O_n   = alpha * O_{n-1} + sum_j exp(s_j - m_n) v_j
and at the end out = O / l, lse = m + ln l.  A row with nothing visible yet
keeps m = -inf; its rescale factor is taken as 0 (nothing to rescale).
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask
from .cu_seqlens import check_cu_seqlens


def _rows_online(Qb, Kb, Vb, vis, scale, block_n):
    rows, D = Qb.shape[0], Vb.shape[1]
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    O = np.zeros((rows, D))
    for n0 in range(0, Kb.shape[0], block_n):
        n1 = min(Kb.shape[0], n0 + block_n)
        s = scale * (Qb @ Kb[n0:n1].T)
        s = np.where(vis[:, n0:n1], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1, initial=-np.inf))
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        p = np.exp(s - safe[:, None])
        l = alpha * l + p.sum(axis=1)
        O = alpha[:, None] * O + p @ Vb[n0:n1]
        m = m_new
    out = np.zeros((rows, D))
    lse = np.full(rows, -np.inf)
    ok = l > 0
    out[ok] = O[ok] / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return out, lse


def _rows_blockwise_normalised(Qb, Kb, Vb, vis, scale, block_n):
    """The computation the pages warn against: softmax per key block, then add."""
    rows, D = Qb.shape[0], Vb.shape[1]
    out = np.zeros((rows, D))
    for n0 in range(0, Kb.shape[0], block_n):
        n1 = min(Kb.shape[0], n0 + block_n)
        s = scale * (Qb @ Kb[n0:n1].T)
        s = np.where(vis[:, n0:n1], s, -np.inf)
        mx = s.max(axis=1, initial=-np.inf)
        safe = np.where(np.isfinite(mx), mx, 0.0)
        p = np.exp(s - safe[:, None])
        l = p.sum(axis=1)
        ok = l > 0
        out[ok] += (p[ok] @ Vb[n0:n1]) / l[ok, None]
    return out


def _per_sequence(q, k, v, cu_q, cu_k, scale, causal, block_n, fn):
    Tq, H, D = q.shape
    cq = check_cu_seqlens(cu_q, Tq)
    ck = check_cu_seqlens(cu_k, k.shape[0])
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((H, Tq), np.nan)
    for b in range(cq.size - 1):
        q0, Lq = int(cq[b]), int(cq[b + 1] - cq[b])
        k0, Lk = int(ck[b]), int(ck[b + 1] - ck[b])
        if Lq == 0:
            continue
        vis = visible_mask(Lq, Lk, causal)
        for h in range(H):
            Qb = q[q0:q0 + Lq, h].astype(np.float64)
            Kb = k[k0:k0 + Lk, h].astype(np.float64)
            Vb = v[k0:k0 + Lk, h].astype(np.float64)
            res = fn(Qb, Kb, Vb, vis, scale, block_n)
            if isinstance(res, tuple):
                out[q0:q0 + Lq, h], lse[h, q0:q0 + Lq] = res
            else:
                out[q0:q0 + Lq, h] = res
    return out, lse


def online_softmax_attention(q, k, v, cu_q, cu_k, scale, causal, block_n=64):
    """Attention by streaming key blocks of ``block_n`` with an online softmax."""
    return _per_sequence(q, k, v, cu_q, cu_k, scale, causal, block_n, _rows_online)


def blockwise_normalised_attention(q, k, v, cu_q, cu_k, scale, causal, block_n=64):
    """Each key block normalised on its own, results added (not attention)."""
    out, _ = _per_sequence(q, k, v, cu_q, cu_k, scale, causal, block_n,
                           _rows_blockwise_normalised)
    return out
