"""Pins for the backward oracle (oracle.attention_grad), CPU, float64.

Each check ties the gradients to something other than the formulas they are
computed with:
  * central finite differences of the forward definition (oracle.attention)
    on tiny ragged inputs, causal and not, with shared key/value heads;
  * a library routine: torch autograd (float64, CPU) through a dense masked
    softmax attention written independently here;
  * invariants of softmax attention: shifting every key by one vector leaves
    each row's softmax unchanged, so the key gradients of a sequence sum to
    zero; probability rows sum to one, so the value gradients of a sequence
    sum to the output gradients of its rows that see a key; a row with a
    single visible key has a constant output, so its query gradient is zero;
  * subsets of heads and sequences agree with the full computation.
Planted mistakes in the oracle (on the CPU) show that the pins catch a
dropped softmax-Jacobian term, a misplaced scale and a wrong head grouping.
"""
import numpy as np
import pytest

import oracle.attention_grad as obwd
from fa_synth import cu_from_lengths
from oracle import attention_bwd, attention_loss, visible_mask

torch = pytest.importorskip("torch")


def rand_case(rng, lq, lk, H, Hk, D):
    cu_q = cu_from_lengths(lq)
    cu_k = cu_from_lengths(lk)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q = rng.standard_normal((Tq, H, D))
    k = rng.standard_normal((Tk, Hk, D))
    v = rng.standard_normal((Tk, Hk, D))
    do = rng.standard_normal((Tq, H, D))
    return q, k, v, do, cu_q, cu_k


def finite_difference(q, k, v, do, cu_q, cu_k, scale, causal, h=1e-6):
    grads = []
    for which in range(3):
        x = [q, k, v][which]
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = attention_loss(*args, do, cu_q, cu_k, scale, causal)
            args[which][idx] -= 2 * h
            lm = attention_loss(*args, do, cu_q, cu_k, scale, causal)
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


FD_CASES = [
    # (lengths_q, lengths_k, H, Hk, D, causal)
    ([3, 5], [4, 2], 2, 1, 4, False),
    ([3, 5], [4, 2], 2, 1, 4, True),
    ([4, 0, 2], [2, 3, 2], 2, 2, 3, True),   # Lq > Lk rows with no key, an empty query side
    ([1, 6], [1, 6], 4, 2, 2, True),
]


@pytest.mark.parametrize("lq,lk,H,Hk,D,causal", FD_CASES)
def test_gradients_match_finite_differences(lq, lk, H, Hk, D, causal):
    rng = np.random.default_rng(len(lq) * 10 + H + D + int(causal))
    q, k, v, do, cu_q, cu_k = rand_case(rng, lq, lk, H, Hk, D)
    scale = 0.7
    dq, dk, dv = attention_bwd(q, k, v, do, cu_q, cu_k, scale, causal)
    fq, fk, fv = finite_difference(q, k, v, do, cu_q, cu_k, scale, causal)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.allclose(got, want, rtol=1e-6, atol=1e-7), np.abs(got - want).max()


def torch_dense_grads(q, k, v, do, cu_q, cu_k, scale, causal):
    """Autograd through softmax(scale q k^T + mask) v, one sequence at a time,
    key/value heads repeated to the query heads."""
    q_t = torch.tensor(q, requires_grad=True)
    k_t = torch.tensor(k, requires_grad=True)
    v_t = torch.tensor(v, requires_grad=True)
    group = q.shape[1] // k.shape[1]
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        Q = q_t[q0:q1].transpose(0, 1)                                   # [H, Lq, D]
        K = k_t[k0:k1].repeat_interleave(group, dim=1).transpose(0, 1)   # [H, Lk, D]
        V = v_t[k0:k1].repeat_interleave(group, dim=1).transpose(0, 1)
        S = scale * torch.matmul(Q, K.transpose(1, 2).contiguous())
        vis = torch.tensor(visible_mask(q1 - q0, k1 - k0, causal))
        rows = vis.any(dim=1)
        S = S.masked_fill(~vis, float("-inf"))
        P = torch.softmax(S[:, rows], dim=-1)
        O = torch.matmul(P, V)
        loss = loss + (torch.tensor(do[q0:q1]).transpose(0, 1)[:, rows] * O).sum()
    loss.backward()
    return [t.grad.numpy() if t.grad is not None else np.zeros(t.shape) for t in (q_t, k_t, v_t)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hk", [(4, 4), (4, 2), (4, 1)])
def test_gradients_match_torch_autograd(causal, H, Hk):
    rng = np.random.default_rng(100 + H * 3 + Hk + int(causal))
    q, k, v, do, cu_q, cu_k = rand_case(rng, [37, 1, 64, 20], [30, 5, 64, 45], H, Hk, 16)
    scale = 0.25
    got = attention_bwd(q, k, v, do, cu_q, cu_k, scale, causal, row_chunk=16)
    want = torch_dense_grads(q, k, v, do, cu_q, cu_k, scale, causal)
    for g, w in zip(got, want):
        assert np.allclose(g, w, rtol=1e-10, atol=1e-12), np.abs(g - w).max()


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    rng = np.random.default_rng(7 + int(causal))
    lq, lk = [50, 9, 70, 0], [40, 9, 90, 5]
    H, Hk, D = 4, 2, 8
    q, k, v, do, cu_q, cu_k = rand_case(rng, lq, lk, H, Hk, D)
    dq, dk, dv = attention_bwd(q, k, v, do, cu_q, cu_k, 0.35, causal)
    group = H // Hk
    for b in range(len(lq)):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        vis = visible_mask(q1 - q0, k1 - k0, causal)
        seen = vis.any(axis=1)
        for hk in range(Hk):
            # key shift invariance: sum over keys of dk is zero
            assert np.allclose(dk[k0:k1, hk].sum(axis=0), 0.0, atol=1e-10)
            # probabilities sum to one: sum over keys of dv = sum of dout over rows that see a key
            want = do[q0:q1][seen][:, hk * group:(hk + 1) * group].sum(axis=(0, 1))
            assert np.allclose(dv[k0:k1, hk].sum(axis=0), want, atol=1e-10)
        # rows with exactly one visible key, or none, pass no query gradient
        one_or_none = vis.sum(axis=1) <= 1
        assert np.allclose(dq[q0:q1][one_or_none], 0.0, atol=1e-12)
    # keys of a sequence without queries are seen by nobody: zero gradients
    b = 3
    assert lq[b] == 0 and lk[b] > 0
    assert np.all(dk[cu_k[b]:cu_k[b + 1]] == 0) and np.all(dv[cu_k[b]:cu_k[b + 1]] == 0)


def test_subsets_agree_with_full():
    rng = np.random.default_rng(11)
    q, k, v, do, cu_q, cu_k = rand_case(rng, [20, 33, 7], [25, 33, 3], 4, 2, 8)
    full = attention_bwd(q, k, v, do, cu_q, cu_k, 0.3, True)
    part = attention_bwd(q, k, v, do, cu_q, cu_k, 0.3, True, heads=[2, 3], seqs=[1])
    sl_q = slice(cu_q[1], cu_q[2])
    sl_k = slice(cu_k[1], cu_k[2])
    assert np.allclose(part[0][sl_q, 2:4], full[0][sl_q, 2:4], rtol=1e-12, atol=1e-14)
    assert np.allclose(part[1][sl_k, 1], full[1][sl_k, 1], rtol=1e-12, atol=1e-14)
    assert np.allclose(part[2][sl_k, 1], full[2][sl_k, 1], rtol=1e-12, atol=1e-14)
    assert np.isnan(part[0][sl_q, 0]).all() and np.isnan(part[1][: cu_k[1]]).all()


def test_shape_errors():
    rng = np.random.default_rng(0)
    q, k, v, do, cu_q, cu_k = rand_case(rng, [3], [3], 2, 1, 4)
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, do[:, :1], cu_q, cu_k, 1.0, False)   # dout shape
    with pytest.raises(ValueError):
        bad = np.zeros((3, 3, 4))
        attention_bwd(q, bad, bad, do, cu_q, cu_k, 1.0, False)       # 3 kv heads do not divide 2


# ---------------------------------------------------------------- planted mistakes
def _fd_pin_passes(lq, lk, H, Hk, D, causal):
    try:
        test_gradients_match_finite_differences(lq, lk, H, Hk, D, causal)
        return True
    except AssertionError:
        return False


def test_planted_dropped_jacobian_term_is_caught(monkeypatch):
    monkeypatch.setattr(obwd, "_softmax_grad", lambda P, dP: P * dP)
    assert not _fd_pin_passes(*FD_CASES[0])


def test_planted_transposed_jacobian_is_caught(monkeypatch):
    monkeypatch.setattr(obwd, "_softmax_grad", lambda P, dP: P * (dP - (P * dP).sum(axis=0, keepdims=True)))
    assert not _fd_pin_passes(*FD_CASES[1])


def test_planted_missing_scale_is_caught(monkeypatch):
    monkeypatch.setattr(obwd, "_input_grads", lambda dS, Q, K, scale: (scale * (dS @ K), dS.T @ Q))
    assert not _fd_pin_passes(*FD_CASES[0])


def test_planted_interleaved_head_grouping_is_caught(monkeypatch):
    rng = np.random.default_rng(5)
    args = rand_case(rng, [9, 12], [9, 12], 4, 2, 4)
    want = torch_dense_grads(*args, 0.5, True)
    got = attention_bwd(*args, 0.5, True)
    assert all(np.allclose(g, w, rtol=1e-10, atol=1e-12) for g, w in zip(got, want))
    monkeypatch.setattr(obwd, "_kv_head", lambda h, H, Hk: h % Hk)
    got = attention_bwd(*args, 0.5, True)
    assert not all(np.allclose(g, w, rtol=1e-10, atol=1e-12) for g, w in zip(got, want))
