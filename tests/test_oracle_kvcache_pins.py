"""Pins for the key/value-cache oracle (oracle.kvcache), CPU, float64.

  * closed form: with all-zero keys every visible key gets the same weight,
    so with one-hot values the output is 1/L at exactly the cache positions
    leftpad_k .. seqlens_k-1 of the sequence (pins which positions are used);
  * a paged cache built here by scattering a plain cache's rows into
    shuffled blocks gives the same result as the plain cache;
  * brute force: keys and values copied position by position with Python
    loops into packed tensors, then the forward definition;
  * one query token under the causal mask sees every cached key (equals the
    non-causal result); shifting the cache contents right by s together with
    leftpad_k and seqlens_k leaves the result unchanged;
  * invalid lengths are rejected.
A planted off-by-one in the cache positions must fail the closed form.
"""
import numpy as np
import pytest

import oracle.kvcache as okv
from fa_synth import cu_from_lengths
from oracle import attention_fwd, attention_kvcache


def make_case(rng, lq, seqlens, leftpad, rows, H=4, Hk=2, D=8):
    B = len(lq)
    cu_q = cu_from_lengths(lq)
    q = rng.standard_normal((int(cu_q[-1]), H, D))
    kc = rng.standard_normal((B, rows, Hk, D))
    vc = rng.standard_normal((B, rows, Hk, D))
    return q, kc, vc, cu_q, np.array(seqlens), (None if leftpad is None else np.array(leftpad))


def test_closed_form_positions():
    B, rows, Hk, H = 3, 13, 1, 2
    lq, seqlens, leftpad = [1, 2, 1], [7, 12, 3], [2, 0, 3]
    D = rows  # one-hot values: V[b, p] = e_p
    cu_q = cu_from_lengths(lq)
    q = np.ones((int(cu_q[-1]), H, D))
    kc = np.zeros((B, rows, Hk, D))
    vc = np.zeros((B, rows, Hk, D))
    for p in range(rows):
        vc[:, p, :, p] = 1.0
    out, lse = attention_kvcache(q, kc, vc, cu_q, seqlens, 0.5, False, leftpad_k=leftpad)
    for b in range(B):
        L = seqlens[b] - leftpad[b]
        want = np.zeros(D)
        want[leftpad[b]:seqlens[b]] = 1.0 / L if L else 0.0
        for i in range(cu_q[b], cu_q[b + 1]):
            assert np.allclose(out[i, 0], want, atol=1e-15)
            assert (lse[0, i] == -np.inf) if L == 0 else np.isclose(lse[0, i], np.log(L))


def scatter_to_pages(rng, cache, page_size, extra_blocks=3):
    """A paged copy of a plain cache: each slot's pages land in shuffled blocks."""
    B, rows = cache.shape[:2]
    per = -(-rows // page_size)
    nblk = B * per + extra_blocks
    order = rng.permutation(nblk)
    table = np.zeros((B, per), dtype=np.int64)
    paged = rng.standard_normal((nblk, page_size) + cache.shape[2:])  # garbage everywhere else
    n = 0
    for b in range(B):
        for j in range(per):
            blk = order[n]
            n += 1
            table[b, j] = blk
            for r in range(page_size):
                p = j * page_size + r
                if p < rows:
                    paged[blk, r] = cache[b, p]
    return paged, table


@pytest.mark.parametrize("causal", [False, True])
def test_paged_equals_plain(causal):
    rng = np.random.default_rng(1)
    q, kc, vc, cu_q, seqlens, leftpad = make_case(rng, [1, 3, 2, 1], [30, 17, 32, 5], [4, 0, 9, 5], 32)
    plain = attention_kvcache(q, kc, vc, cu_q, seqlens, 0.3, causal, leftpad_k=leftpad)
    pk, table = scatter_to_pages(np.random.default_rng(2), kc, 8)
    pv, _ = scatter_to_pages(np.random.default_rng(2), vc, 8)
    paged = attention_kvcache(q, pk, pv, cu_q, seqlens, 0.3, causal, leftpad_k=leftpad, block_table=table,
                              page_size=8)
    assert np.array_equal(plain[0], paged[0], equal_nan=True)
    assert np.array_equal(plain[1], paged[1])


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_gather(causal):
    rng = np.random.default_rng(3)
    q, kc, vc, cu_q, seqlens, leftpad = make_case(rng, [2, 1, 4], [20, 9, 31], [3, 0, 1], 31)
    ks, vs, lens = [], [], []
    for b in range(3):
        for p in range(leftpad[b], seqlens[b]):
            ks.append(kc[b, p])
            vs.append(vc[b, p])
        lens.append(seqlens[b] - leftpad[b])
    want = attention_fwd(q, np.array(ks), np.array(vs), cu_q, cu_from_lengths(lens), 0.25, causal)
    got = attention_kvcache(q, kc, vc, cu_q, seqlens, 0.25, causal, leftpad_k=leftpad)
    assert np.allclose(got[0], want[0], rtol=1e-13, atol=1e-14)
    assert np.allclose(got[1], want[1], rtol=1e-13, atol=1e-14)


def test_single_token_causal_sees_all_and_shift_invariance():
    rng = np.random.default_rng(4)
    q, kc, vc, cu_q, seqlens, leftpad = make_case(rng, [1, 1, 1], [10, 25, 7], [0, 5, 2], 40)
    a = attention_kvcache(q, kc, vc, cu_q, seqlens, 0.4, True, leftpad_k=leftpad)
    b = attention_kvcache(q, kc, vc, cu_q, seqlens, 0.4, False, leftpad_k=leftpad)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    s = 6
    kc2 = np.zeros_like(kc)
    vc2 = np.zeros_like(vc)
    kc2[:, s:] = kc[:, :-s]
    vc2[:, s:] = vc[:, :-s]
    c = attention_kvcache(q, kc2, vc2, cu_q, seqlens + s, 0.4, True, leftpad_k=leftpad + s)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_invalid_lengths():
    rng = np.random.default_rng(5)
    q, kc, vc, cu_q, seqlens, _ = make_case(rng, [1, 1], [5, 8], None, 8)
    with pytest.raises(ValueError):
        attention_kvcache(q, kc, vc, cu_q, np.array([5, 9]), 0.5, False)         # longer than the slot
    with pytest.raises(ValueError):
        attention_kvcache(q, kc, vc, cu_q, seqlens, 0.5, False, leftpad_k=np.array([6, 0]))
    with pytest.raises(ValueError):
        attention_kvcache(q, kc, vc, cu_q, np.array([5]), 0.5, False)            # one length per sequence


def test_planted_off_by_one_positions_is_caught(monkeypatch):
    real = okv.cache_positions
    monkeypatch.setattr(okv, "cache_positions",
                        lambda batch, s, lp=None: [p + 1 for p in real(batch, s, lp)])
    with pytest.raises(AssertionError):
        test_closed_form_positions()
