"""Pins for the oracle: each check ties it to something other than itself.

Kinds of pin used here (all CPU, float64):
  * values printed on the pages (cu_seqlens worked examples, tests/golden/);
  * closed forms (one key, causal first row, equal scores, all-ones values);
  * invariants (shift of K, affine map of V, joint permutation of K/V rows,
    packing equals running each sequence alone);
  * brute force with math.fsum on tiny inputs;
  * a library routine on the special cases it covers (torch SDPA, scipy
    logsumexp);
  * the pages' equivalence claim (online softmax equals the global softmax;
    per-block normalise-then-add does not).
The planted-mistake tests at the end show that plausible errors in the oracle
fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import oracle.attention as oatt
from oracle import (attention_fwd, attention_rows, blockwise_normalised_attention, check_cu_seqlens,
                    flops_visible_pairs, lengths_from_cu, online_softmax_attention, row_offset,
                    tile_items, tile_map)
from fa_synth import cu_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(rng, lq, lk, H, D):
    cu_q = cu_from_lengths(lq)
    cu_k = cu_from_lengths(lk)
    q = rng.standard_normal((int(cu_q[-1]), H, D))
    k = rng.standard_normal((int(cu_k[-1]), H, D))
    v = rng.standard_normal((int(cu_k[-1]), H, D))
    return q, k, v, cu_q, cu_k


# ---------------------------------------------------------------- cu_seqlens
def test_worked_examples_lengths():
    with open(os.path.join(GOLDEN, "cu_seqlens_worked_examples.json")) as f:
        g = json.load(f)
    assert len(g["cases"]) == 3
    for case in g["cases"]:
        assert lengths_from_cu(case["cu_seqlens"]).tolist() == case["lengths"]


def test_cu_seqlens_validity():
    with pytest.raises(ValueError):
        check_cu_seqlens([1, 2, 3])
    with pytest.raises(ValueError):
        check_cu_seqlens([0, 5, 4])
    with pytest.raises(ValueError):
        check_cu_seqlens([0, 5, 10], total_rows=9)
    assert check_cu_seqlens([0]).tolist() == [0]
    assert lengths_from_cu([0, 0, 7, 7]).tolist() == [0, 7, 0]


def test_row_offset_is_start_times_row_stride():
    # sequence 1 of [0,128,300] starts at row 128 of a [300, 12, 64] packed tensor
    assert row_offset([0, 128, 300], 1, 12 * 64) == 128 * 12 * 64
    assert row_offset([0, 128, 300], 0, 12 * 64) == 0


# ---------------------------------------------------------------- tile map
def test_tile_map_worked_examples():
    assert tile_map([0, 128, 300], 128).tolist() == [0, 1, 3]
    assert tile_map([0, 200, 1024], 128).tolist() == [0, 2, 9]
    assert tile_map([0, 200, 1024], 64).tolist() == [0, 4, 17]
    assert tile_map([0, 0, 5, 5, 300], 128).tolist() == [0, 0, 1, 1, 4]
    assert tile_items([0, 128, 300], 128).tolist() == [[0, 0], [1, 0], [1, 1]]


def _check_tile_cover(cu, bm):
    cu = np.asarray(cu, dtype=np.int64)
    bs = tile_map(cu, bm)
    items = tile_items(cu, bm)
    lens = cu[1:] - cu[:-1]
    assert bs[0] == 0 and bs[-1] == items.shape[0]
    assert int(bs[-1]) == int(sum(-(-int(L) // bm) for L in lens))
    hits = np.zeros(int(cu[-1]), dtype=np.int64)
    prev = (-1, -1)
    for t, (b, m) in enumerate(items):
        assert bs[b] <= t < bs[b + 1]
        assert (b, m) > prev  # sequence-major, block-ascending
        prev = (b, m)
        r0 = cu[b] + m * bm
        r1 = min(cu[b + 1], cu[b] + (m + 1) * bm)
        assert cu[b] <= r0 < r1 <= cu[b + 1]  # non-empty, never straddles a sequence
        hits[r0:r1] += 1
    assert np.all(hits == 1)  # every packed row covered exactly once


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 700), min_size=1, max_size=12), st.sampled_from([1, 16, 64, 128, 256]))
def test_tile_map_covers_rows_once(lengths, bm):
    _check_tile_cover(cu_from_lengths(lengths), bm)


# ---------------------------------------------------------------- attention pins
def pin_ones_v(attn):
    rng = np.random.default_rng(1)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [5, 9, 3], [7, 4, 3], 2, 8)
    v = np.ones_like(v)
    ok = True
    for causal in (False, True):
        out, lse = attn(q, k, v, cu_q, cu_k, 0.4, causal)
        has = np.isfinite(lse.T)  # [Tq, H]
        ok &= np.allclose(out[has], 1.0, atol=1e-13, rtol=0)
        ok &= np.all(out[~has] == 0.0)
    return bool(ok)


def pin_one_key(attn):
    rng = np.random.default_rng(2)
    lq = [4, 6, 1]
    q, k, v, cu_q, cu_k = rand_qkv(rng, lq, [1, 1, 1], 3, 5)
    scale = 0.7
    out, lse = attn(q, k, v, cu_q, cu_k, scale, False)
    ok = True
    for b in range(3):
        for i in range(cu_q[b], cu_q[b + 1]):
            for h in range(3):
                ok &= np.allclose(out[i, h], v[cu_k[b], h], atol=1e-13, rtol=0)
                ok &= abs(lse[h, i] - scale * q[i, h] @ k[cu_k[b], h]) < 1e-12
    # causal with one key: only the last query row of each sequence sees it
    out, lse = attn(q, k, v, cu_q, cu_k, scale, True)
    for b in range(3):
        last = cu_q[b + 1] - 1
        for h in range(3):
            ok &= np.allclose(out[last, h], v[cu_k[b], h], atol=1e-13, rtol=0)
            for i in range(cu_q[b], last):
                ok &= np.all(out[i, h] == 0) and lse[h, i] == -np.inf
    return bool(ok)


def pin_causal_first_row(attn):
    rng = np.random.default_rng(3)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [6, 11], [6, 11], 2, 7)
    scale = 0.3
    out, lse = attn(q, k, v, cu_q, cu_k, scale, True)
    ok = True
    for b in range(2):
        i0, j0 = cu_q[b], cu_k[b]
        for h in range(2):
            ok &= np.allclose(out[i0, h], v[j0, h], atol=1e-13, rtol=0)
            ok &= abs(lse[h, i0] - scale * q[i0, h] @ k[j0, h]) < 1e-12
    return bool(ok)


def pin_equal_scores(attn):
    """Q = 0: every visible key scores 0, so out is the mean of the visible
    values and lse = ln(#visible).  Causal (bottom-right) row i of a sequence
    sees the first clip(i + Lk - Lq + 1, 0, Lk) keys."""
    rng = np.random.default_rng(4)
    lq, lk = [5, 9, 3, 4], [8, 4, 3, 0]
    q, k, v, cu_q, cu_k = rand_qkv(rng, lq, lk, 2, 6)
    q = np.zeros_like(q)
    ok = True
    for causal in (False, True):
        out, lse = attn(q, k, v, cu_q, cu_k, 1.3, causal)
        for b in range(len(lq)):
            Lq, Lk = lq[b], lk[b]
            Vb = v[cu_k[b]:cu_k[b + 1]]
            prefix = np.concatenate([np.zeros((1,) + Vb.shape[1:]), np.cumsum(Vb, axis=0)])
            for i in range(Lq):
                n = Lk if not causal else min(Lk, max(0, i + Lk - Lq + 1))
                row = cu_q[b] + i
                for h in range(2):
                    if n == 0:
                        ok &= np.all(out[row, h] == 0) and lse[h, row] == -np.inf
                    else:
                        ok &= np.allclose(out[row, h], prefix[n, h] / n, atol=1e-13, rtol=0)
                        ok &= abs(lse[h, row] - math.log(n)) < 1e-13
    return bool(ok)


def brute_force(q, k, v, cu_q, cu_k, scale, causal):
    """Pure-Python triple loop, exp and math.fsum; tiny inputs only."""
    Tq, H, D = q.shape
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((H, Tq), np.nan)
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for h in range(H):
            for i in range(Lq):
                qi = q[cu_q[b] + i, h]
                scores = []
                for j in range(Lk):
                    if causal and j > i + Lk - Lq:
                        continue
                    kj = k[cu_k[b] + j, h]
                    scores.append((j, scale * math.fsum(float(qi[d]) * float(kj[d]) for d in range(D))))
                row = cu_q[b] + i
                if not scores:
                    out[row, h] = 0.0
                    lse[h, row] = -math.inf
                    continue
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                den = math.fsum(e for _, e in w)
                for d in range(D):
                    out[row, h, d] = math.fsum(e * float(v[cu_k[b] + j, h, d]) for j, e in w) / den
                lse[h, row] = mx + math.log(den)
    return out, lse


def pin_brute_force(attn):
    rng = np.random.default_rng(5)
    ok = True
    for trial in range(12):
        B = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(0, 9, size=B)]
        lk = [int(x) for x in rng.integers(0, 9, size=B)]
        H, D = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        q, k, v, cu_q, cu_k = rand_qkv(rng, lq, lk, H, D)
        for causal in (False, True):
            scale = float(rng.uniform(0.1, 2.0))
            o1, s1 = attn(q, k, v, cu_q, cu_k, scale, causal)
            o2, s2 = brute_force(q, k, v, cu_q, cu_k, scale, causal)
            ok &= np.allclose(o1, o2, atol=1e-12, rtol=0, equal_nan=True)
            fin = np.isfinite(s2)
            ok &= np.array_equal(np.isfinite(s1), fin) and np.array_equal(np.isnan(s1), np.isnan(s2))
            ok &= np.allclose(s1[fin], s2[fin], atol=1e-12, rtol=0)
            ok &= np.array_equal(s1[np.isinf(s2)], s2[np.isinf(s2)])
    return bool(ok)


def pin_packed_equals_alone(attn):
    rng = np.random.default_rng(6)
    lq, lk = [7, 0, 12, 5], [9, 3, 12, 2]
    q, k, v, cu_q, cu_k = rand_qkv(rng, lq, lk, 2, 4)
    ok = True
    for causal in (False, True):
        out, lse = attn(q, k, v, cu_q, cu_k, 0.5, causal)
        for b in range(4):
            qs = q[cu_q[b]:cu_q[b + 1]]
            ks, vs = k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]]
            o1, s1 = attn(qs, ks, vs, [0, lq[b]], [0, lk[b]], 0.5, causal)
            ok &= np.allclose(out[cu_q[b]:cu_q[b + 1]], o1, atol=1e-14, rtol=0)
            ok &= np.array_equal(lse[:, cu_q[b]:cu_q[b + 1]], s1) or np.allclose(
                lse[:, cu_q[b]:cu_q[b + 1]], s1, atol=1e-14, rtol=0)
    return bool(ok)


def pin_invariances(attn):
    rng = np.random.default_rng(7)
    lq, lk = [6, 10], [9, 10]
    H, D = 2, 5
    q, k, v, cu_q, cu_k = rand_qkv(rng, lq, lk, H, D)
    scale = 0.6
    ok = True
    for causal in (False, True):
        out, lse = attn(q, k, v, cu_q, cu_k, scale, causal)
        # shift every key by u (per head): scores gain scale*q.u uniformly per row
        u = rng.standard_normal((H, D))
        o2, s2 = attn(q, k + u[None], v, cu_q, cu_k, scale, causal)
        fin = np.isfinite(lse)
        ok &= np.allclose(o2, out, atol=1e-12, rtol=0, equal_nan=True)
        expect = lse + scale * np.einsum("thd,hd->ht", q, u)
        ok &= np.allclose(s2[fin], expect[fin], atol=1e-12, rtol=0)
        # affine map of values: out -> out A + c on rows with visible keys
        A = rng.standard_normal((H, D, D))
        c = rng.standard_normal((H, D))
        o3, _ = attn(q, k, np.einsum("thd,hde->the", v, A) + c[None], cu_q, cu_k, scale, causal)
        exp3 = np.einsum("thd,hde->the", out, A) + c[None]
        has = fin.T
        ok &= np.allclose(o3[has], exp3[has], atol=1e-12, rtol=0)
    # joint permutation of key/value rows inside each sequence: non-causal only
    out, lse = attn(q, k, v, cu_q, cu_k, scale, False)
    perm = np.concatenate([cu_k[b] + rng.permutation(lk[b]) for b in range(2)])
    o4, s4 = attn(q, k[perm], v[perm], cu_q, cu_k, scale, False)
    ok &= np.allclose(o4, out, atol=1e-12, rtol=0) and np.allclose(s4, lse, atol=1e-12, rtol=0)
    return bool(ok)


def pin_stability(attn):
    """Huge scale: softmax becomes argmax; nothing overflows to NaN or Inf."""
    rng = np.random.default_rng(8)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [16], [16], 1, 8)
    out, lse = attn(q, k, v, cu_q, cu_k, 50.0, False)
    ok = bool(np.all(np.isfinite(out)) and np.all(np.isfinite(lse)))
    s = q[:, 0] @ k[:, 0].T
    for i in range(16):
        srt = np.sort(s[i])
        if 50.0 * (srt[-1] - srt[-2]) > 40:  # winner clear by e^-40
            ok &= np.allclose(out[i, 0], v[np.argmax(s[i]), 0], atol=1e-12, rtol=0)
    return ok


def pin_library(attn):
    """Special cases a library routine covers: torch SDPA (float64, CPU) per
    sequence, non-causal and causal with Lq == Lk (where its top-left causal
    mask coincides with bottom-right); scipy's logsumexp for lse."""
    import torch
    from scipy.special import logsumexp
    rng = np.random.default_rng(9)
    lens = [13, 40, 1, 27]
    q, k, v, cu_q, cu_k = rand_qkv(rng, lens, lens, 3, 16)
    scale = 0.25
    ok = True
    for causal in (False, True):
        out, lse = attn(q, k, v, cu_q, cu_k, scale, causal)
        for b in range(len(lens)):
            sl = slice(cu_q[b], cu_q[b + 1])
            tq = torch.from_numpy(q[sl]).permute(1, 0, 2)
            tk = torch.from_numpy(k[sl]).permute(1, 0, 2)
            tv = torch.from_numpy(v[sl]).permute(1, 0, 2)
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, is_causal=causal, scale=scale).permute(1, 0, 2).numpy()
            ok &= np.allclose(out[sl], ref, atol=1e-12, rtol=0)
            S = scale * np.einsum("ihd,jhd->hij", q[sl], k[sl])
            if causal:
                S = np.where(np.tril(np.ones(S.shape[1:], dtype=bool))[None], S, -np.inf)
            ok &= np.allclose(lse[:, sl], logsumexp(S, axis=2), atol=1e-12, rtol=0)
    return bool(ok)


PINS = [pin_ones_v, pin_one_key, pin_causal_first_row, pin_equal_scores, pin_brute_force,
        pin_packed_equals_alone, pin_invariances, pin_stability, pin_library]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    assert pin(attention_fwd)


def test_fully_masked_rows_exact():
    """Causal, Lq > Lk: the first Lq - Lk rows see nothing -> exactly 0 / -inf."""
    rng = np.random.default_rng(10)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [824, 5], [724, 0], 2, 8)
    out, lse = attention_fwd(q, k, v, cu_q, cu_k, 0.125, True)
    assert np.all(out[:100] == 0) and np.all(lse[:, :100] == -np.inf)
    assert np.all(np.isfinite(out[100:824])) and np.all(np.isfinite(lse[:, 100:824]))
    assert np.all(out[824:829] == 0) and np.all(lse[:, 824:829] == -np.inf)


def test_rows_outside_sequences_are_nan():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((10, 1, 4))
    k = rng.standard_normal((10, 1, 4))
    out, lse = attention_fwd(q, k, k, [0, 6], [0, 6], 1.0, False)
    assert np.all(np.isnan(out[6:])) and np.all(np.isnan(lse[:, 6:]))
    assert np.all(np.isfinite(out[:6]))


def test_attention_rows_matches_full():
    rng = np.random.default_rng(12)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [50, 130, 7], [60, 130, 2], 3, 16)
    for causal in (False, True):
        out, lse = attention_fwd(q, k, v, cu_q, cu_k, 0.25, causal)
        rows = [0, 3, 49, 50, 100, 179, 180, 186]
        heads = [2, 0]
        o, s = attention_rows(q, k, v, cu_q, cu_k, 0.25, causal, rows, heads)
        assert np.allclose(o, out[rows][:, heads], atol=1e-14, rtol=0)
        assert np.allclose(s, lse[heads][:, rows], atol=1e-14, rtol=0)


def test_visible_pair_counts_closed_forms():
    # non-causal: sum Lq*Lk; causal Lq == Lk: L(L+1)/2; causal Lq > Lk: rows below the shift see nothing
    assert flops_visible_pairs([0, 128, 300], [0, 128, 300], False) == 128 * 128 + 172 * 172
    assert flops_visible_pairs([0, 2048], [0, 2048], True) == 2048 * 2049 // 2
    # Lq=824, Lk=724: row i sees clip(i - 99, 0, 724) keys
    expect = sum(min(724, max(0, i - 100 + 1)) for i in range(824))
    assert flops_visible_pairs([0, 824], [0, 724], True) == expect
    # Lq=200, Lk=300: row i sees i + 101 keys
    assert flops_visible_pairs([0, 200], [0, 300], True) == sum(i + 101 for i in range(200))


# ---------------------------------------------------------------- online softmax (pages' claim)
@pytest.mark.parametrize("block_n", [1, 3, 16, 64, 1000])
def test_online_softmax_equals_global(block_n):
    rng = np.random.default_rng(13)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [33, 70, 5, 0], [40, 70, 9, 3], 2, 8)
    for causal in (False, True):
        o1, s1 = attention_fwd(q, k, v, cu_q, cu_k, 0.4, causal)
        o2, s2 = online_softmax_attention(q, k, v, cu_q, cu_k, 0.4, causal, block_n)
        assert np.allclose(o1, o2, atol=1e-12, rtol=0, equal_nan=True)
        assert np.allclose(s1, s2, atol=1e-12, rtol=0, equal_nan=True)


def test_blockwise_normalised_is_not_attention():
    rng = np.random.default_rng(14)
    q, k, v, cu_q, cu_k = rand_qkv(rng, [64], [256], 2, 8)
    o1, _ = attention_fwd(q, k, v, cu_q, cu_k, 0.4, False)
    o3 = blockwise_normalised_attention(q, k, v, cu_q, cu_k, 0.4, False, 64)
    assert np.max(np.abs(o1 - o3)) > 1e-2
    # with a single block the two coincide
    o4 = blockwise_normalised_attention(q, k, v, cu_q, cu_k, 0.4, False, 256)
    assert np.allclose(o1, o4, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- planted mistakes
def _mask_top_left(Lq, Lk, causal, rows=None):
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    if not causal:
        return np.ones((i.size, Lk), dtype=bool)
    return np.arange(Lk)[None, :] <= i[:, None]


def _mask_strict(Lq, Lk, causal, rows=None):
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    if not causal:
        return np.ones((i.size, Lk), dtype=bool)
    return np.arange(Lk)[None, :] < i[:, None] + (Lk - Lq)


def _softmax_log2(S, vis, Vb):
    out, lse = _ORIG_SOFTMAX(S, vis, Vb)
    return out, lse / math.log(2.0)


def _softmax_no_max_guard(S, vis, Vb):
    out, lse = _ORIG_SOFTMAX(S, vis, Vb)
    return out, np.where(np.isinf(lse), 0.0, lse)


_ORIG_SOFTMAX = oatt._softmax_rows

MUTANTS = {
    "swap_k_v": lambda q, k, v, cq, ck, s, c: attention_fwd(q, v, k, cq, ck, s, c),
    "drop_scale": lambda q, k, v, cq, ck, s, c: attention_fwd(q, k, v, cq, ck, 1.0, c),
    "k_offsets_from_q": lambda q, k, v, cq, ck, s, c: attention_fwd(
        q, k, v, cq, cq if int(cq[-1]) <= k.shape[0] else ck, s, c),
    "transpose_qk": lambda q, k, v, cq, ck, s, c: attention_fwd(k, q, v, ck, cq, s, c)
    if q.shape == k.shape else attention_fwd(q, k, v, cq, ck, s, c),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_argument_mistakes_fail_a_pin(name):
    fn = MUTANTS[name]
    results = {p.__name__: p(fn) for p in PINS}
    assert not all(results.values()), f"mutant {name} passed every pin"


@pytest.mark.parametrize("patch", ["mask_top_left", "mask_strict", "lse_log2", "empty_row_lse"])
def test_planted_internal_mistakes_fail_a_pin(patch, monkeypatch):
    if patch == "mask_top_left":
        monkeypatch.setattr(oatt, "visible_mask", _mask_top_left)
    elif patch == "mask_strict":
        monkeypatch.setattr(oatt, "visible_mask", _mask_strict)
    elif patch == "lse_log2":
        monkeypatch.setattr(oatt, "_softmax_rows", _softmax_log2)
    elif patch == "empty_row_lse":
        monkeypatch.setattr(oatt, "_softmax_rows", _softmax_no_max_guard)
    results = {p.__name__: p(oatt.attention_fwd) for p in PINS}
    assert not all(results.values()), f"planted mistake {patch} passed every pin"


# ---------------------------------------------------------------- shared key/value heads
def _gqa_case(rng, H=8, Hk=2, D=16):
    cu_q, cu_k = cu_from_lengths([13, 0, 29, 7]), cu_from_lengths([11, 4, 29, 20])
    q = rng.standard_normal((int(cu_q[-1]), H, D))
    k = rng.standard_normal((int(cu_k[-1]), Hk, D))
    v = rng.standard_normal((int(cu_k[-1]), Hk, D))
    return q, k, v, cu_q, cu_k


def pin_gqa_repeat(attn, H=8, Hk=2):
    """Query head h shares key/value head h // (H/Hk): the result equals plain
    multi-head attention on K/V whose heads are repeated H/Hk times each
    (numpy's repeat builds the shared heads independently of the oracle)."""
    rng = np.random.default_rng(40 + Hk)
    q, k, v, cq, ck = _gqa_case(rng, H, Hk)
    ok = True
    for causal in (False, True):
        o, l = attn(q, k, v, cq, ck, 0.3, causal)
        kr, vr = np.repeat(k, H // Hk, axis=1), np.repeat(v, H // Hk, axis=1)
        ro, rl = attention_fwd(q, kr, vr, cq, ck, 0.3, causal)
        n = int(cq[-1])
        ok &= np.array_equal(o[:n], ro[:n]) and np.array_equal(l[:, :n], rl[:, :n])
    return bool(ok)


@pytest.mark.parametrize("Hk", [1, 2, 4, 8])
def test_gqa_equals_mha_on_repeated_heads(Hk):
    assert pin_gqa_repeat(attention_fwd, 8, Hk)


def test_gqa_rows_match_full():
    rng = np.random.default_rng(44)
    q, k, v, cq, ck = _gqa_case(rng, 8, 2)
    rows = [0, 5, 12, 13, 30, 41, 48]
    heads = [0, 3, 4, 7]
    fo, fl = attention_fwd(q, k, v, cq, ck, 0.3, True)
    so, sl = attention_rows(q, k, v, cq, ck, 0.3, True, rows, heads)
    assert np.allclose(so, fo[rows][:, heads], rtol=1e-12, atol=1e-12)
    assert np.allclose(sl, fl[heads][:, rows], rtol=1e-12, atol=1e-12)


def test_gqa_head_count_must_divide():
    rng = np.random.default_rng(45)
    q = rng.standard_normal((4, 6, 8))
    k = rng.standard_normal((4, 4, 8))
    with pytest.raises(ValueError):
        attention_fwd(q, k, k, [0, 4], [0, 4], 1.0, False)
    assert oracle.kv_head_of(32, 8) == 4 and oracle.kv_head_of(5, 1) == 5


def test_planted_gqa_interleaved_mapping_fails(monkeypatch):
    """Pairing query head h with key/value head h % Hk (interleaved instead of
    contiguous groups) must fail the repeat pin."""
    def interleaved(q, k, v, cq, ck, s, c):
        Hk = k.shape[1]
        kk = np.stack([k[:, h % Hk] for h in range(q.shape[1])], axis=1)
        vv = np.stack([v[:, h % Hk] for h in range(q.shape[1])], axis=1)
        return attention_fwd(q, kk, vv, cq, ck, s, c)
    assert not pin_gqa_repeat(interleaved, 8, 2)
