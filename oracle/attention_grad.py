"""Gradients of exact varlen attention (the backward pass), float64.

TEST INFRASTRUCTURE (see the package docstring for who may import it).

What is computed: for a scalar loss whose gradient with respect to the
attention output is ``dout``, the gradients dq, dk and dv of the forward
defined in :mod:`oracle.attention` (same offsets, masks and head grouping).

The pages describe how the tiled backward pass is organised -- each worker
owns a block of key columns, recomputes the attention of its block instead of
storing it, and the workers add their contributions to the query gradient
with atomic operations (zepes.com, "Comprendiendo Flash-Atención y
Flash-Atención-2", section "FashAttention v1" (sic); recomputation and tiling are
named in the same section).  They do not print the gradient formulas.  What
the tiled pass must equal is the derivative of the forward definition, which
follows from the chain rule on the materialised matrices of one (sequence,
head):

    S  = scale * Q K^T           (visible pairs only)
    P  = softmax_rows(S)         O = P V
    dV = P^T dO                  dP = dO V^T
    dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian, row by row)
    dQ = scale * dS K            dK = scale * dS^T Q

Readings:
  * With grouped key/value heads (Hk < H), a key/value head is used by H/Hk
    query heads, so its dk and dv are the sums over those heads.
  * A row with no visible key has the constant output 0 and passes no
    gradient: its dq is 0 and it adds nothing to dk or dv.
  * Keys that no query sees get dk = dv = 0.
  * Inputs are used at the exact values the device receives; all arithmetic
    is float64.  Rows are processed in chunks of at most ``row_chunk`` queries
    (every row is still complete over its keys, so this is the definition).

Layouts: q, dout, dq [Tq, H, D]; k, v, dk, dv [Tk, Hk, D].  Rows outside
every sequence are returned as NaN.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import _check_shapes, visible_mask
from .cu_seqlens import check_cu_seqlens


def _probabilities(S: np.ndarray, vis: np.ndarray) -> np.ndarray:
    """Row softmax over the visible entries; rows with none are all zero."""
    S = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    mu = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.exp(S - mu[:, None])
    l = E.sum(axis=1)
    P = np.zeros_like(S)
    P[any_vis] = E[any_vis] / l[any_vis, None]
    return P


def _softmax_grad(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """Gradient with respect to the scores: the softmax Jacobian applied to dP.

    For p = softmax(s), dp/ds = diag(p) - p p^T, so ds = p * (dp - <p, dp>).
    """
    return P * (dP - (P * dP).sum(axis=1, keepdims=True))


def _input_grads(dS: np.ndarray, Q: np.ndarray, K: np.ndarray, scale: float):
    """dQ and dK from the score gradient: S = scale Q K^T gives dQ = scale dS K
    and dK = scale dS^T Q."""
    return scale * (dS @ K), scale * (dS.T @ Q)


def _kv_head(h: int, H: int, Hk: int) -> int:
    """Key/value head used by query head h: contiguous groups of H/Hk heads."""
    return h // (H // Hk)


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, cu_q, cu_k,
                  scale: float, causal: bool, heads: Optional[Sequence[int]] = None,
                  seqs: Optional[Sequence[int]] = None, row_chunk: int = 1024):
    """dq, dk, dv of exact varlen attention in float64.

    ``heads`` restricts the computation to a subset of query heads and
    ``seqs`` to a subset of sequences; dk and dv of a key/value head are then
    summed over the selected query heads only (pass whole groups to get the
    full gradient).  Entries not computed stay NaN.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    _check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    Tq, H, D = q.shape
    Tk, Hk = k.shape[0], k.shape[1]
    cq = check_cu_seqlens(cu_q, Tq)
    ck = check_cu_seqlens(cu_k, Tk)
    if cq.size != ck.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    hs = list(range(H)) if heads is None else list(heads)
    bs = range(cq.size - 1) if seqs is None else list(seqs)
    dq = np.full((Tq, H, D), np.nan, dtype=np.float64)
    dk = np.full((Tk, Hk, D), np.nan, dtype=np.float64)
    dv = np.full((Tk, Hk, D), np.nan, dtype=np.float64)
    for b in bs:
        q0, Lq = int(cq[b]), int(cq[b + 1] - cq[b])
        k0, Lk = int(ck[b]), int(ck[b + 1] - ck[b])
        for hk in sorted({_kv_head(h, H, Hk) for h in hs}):
            dk[k0:k0 + Lk, hk, :] = 0.0
            dv[k0:k0 + Lk, hk, :] = 0.0
        for h in hs:
            hk = _kv_head(h, H, Hk)
            Kb = k[k0:k0 + Lk, hk, :].astype(np.float64)
            Vb = v[k0:k0 + Lk, hk, :].astype(np.float64)
            for r0 in range(0, Lq, row_chunk):
                r1 = min(Lq, r0 + row_chunk)
                Qb = q[q0 + r0:q0 + r1, h, :].astype(np.float64)
                dOb = dout[q0 + r0:q0 + r1, h, :].astype(np.float64)
                vis = visible_mask(Lq, Lk, causal, np.arange(r0, r1))
                P = _probabilities(scale * (Qb @ Kb.T), vis)
                dS = _softmax_grad(P, dOb @ Vb.T)
                gq, gk = _input_grads(dS, Qb, Kb, scale)
                dq[q0 + r0:q0 + r1, h, :] = gq
                dk[k0:k0 + Lk, hk, :] += gk
                dv[k0:k0 + Lk, hk, :] += P.T @ dOb
    return dq, dk, dv


def attention_loss(q, k, v, dout, cu_q, cu_k, scale: float, causal: bool) -> float:
    """The scalar sum(dout * out) whose gradient attention_bwd returns."""
    from .attention import attention_fwd
    out, _ = attention_fwd(q, k, v, cu_q, cu_k, scale, causal)
    n = int(check_cu_seqlens(cu_q)[-1])
    return float((np.asarray(dout, dtype=np.float64)[:n] * out[:n]).sum())
