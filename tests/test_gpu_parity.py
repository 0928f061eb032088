"""GPU parity: the HIP path, called through the C ABI, against the oracle.

Bar (from the method's exactness up to floating-point order): the work-item
map is bit-exact; out and lse agree to max-abs 2e-2 for bf16 inputs (fp32
accumulation, bf16 probabilities and output) and 1e-5 for fp32 inputs; rows
with no visible key give lse = -inf exactly and out = 0.

Configurations: the tiny fp32 batch, the ragged q/k batch and the dense
8x2048 batch are compared in full; the 16k-token sweep and the ragged 64k
batch (the sizes and launch configuration the bench times) are compared on
sampled rows and heads.  Edge cases: empty sequences, single tokens, ragged
tails, Lq != Lk with causal masks, hundreds of short sequences, poisoned and
guarded output buffers, determinism.
"""
import os

import numpy as np
import pytest

from fa_synth import (SWEEP_HEAD_DIMS, SWEEP_SEQLENS, draw_qkv, workload_custom, workload_dense,
                      workload_ragged64k, workload_ragged64k_gqa, workload_ragged_qk, workload_sweep, workload_tiny)
from oracle import attention_fwd, attention_rows, tile_map
from tests._gpu_util import TOL, compare, dtype_code, host, run_gpu, sample_rows, say, to_device

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def fa():
    import variable_length_flashattention_cu_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback exists
    return m


def full_parity(fa, wl, causal):
    say(f"case {wl.name} causal={causal} dtype={wl.dtype}")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    o, l = host(*run_gpu(wl, t, causal))
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    n = wl.total_q
    return compare(o[:n], l[:, :n], ref_o[:n], ref_l[:, :n], TOL[wl.dtype], wl.name)


# ---------------------------------------------------------------- tile map
def test_tile_map_bit_exact(fa):
    rng = np.random.default_rng(100)
    cases = [[0, 128, 300], [0, 200, 1024], [0, 300, 1024], [0], [0, 0, 0], [0, 5, 5, 300, 300]]
    for _ in range(20):
        lens = rng.integers(0, 700, size=int(rng.integers(1, 40)))
        cases.append([0] + np.cumsum(lens).tolist())
    lens = rng.integers(0, 300, size=1000)  # several scan chunks of 256
    cases.append([0] + np.cumsum(lens).tolist())
    # every block height the forward pass uses (fp32 and 16-bit kernels)
    configs = [(d, dt) for d in (64, 96, 128) for dt in (fa.FA_DTYPE_F32, fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16)]
    configs += [(256, fa.FA_DTYPE_BF16)]
    assert len({fa.fa_varlen_block_sizes(d, dt)[0] for d, dt in configs}) >= 2
    for cu in cases:
        cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
        max_q = int(np.diff(cu).max()) if len(cu) > 1 else 0
        for d, dt in configs:
            bm = fa.fa_varlen_block_sizes(d, dt)[0]
            got = fa.fa_varlen_tile_map(cu_t, max_q, d, dt).cpu().numpy()
            assert np.array_equal(got, tile_map(cu, bm)), (cu[:5], d, dt, bm)


# ---------------------------------------------------------------- configurations, full comparison
def test_tiny_fp32(fa):
    full_parity(fa, workload_tiny(), False)


def test_tiny_fp32_causal(fa):
    full_parity(fa, workload_tiny(), True)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_qk(fa, causal):
    full_parity(fa, workload_ragged_qk(), causal)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_8x2048(fa, causal):
    full_parity(fa, workload_dense(), causal)


# ---------------------------------------------------------------- full sizes, sampled rows
def sampled_parity(fa, wl, causal, heads, seed, full_head=None):
    """Sampled rows of `heads`; with `full_head`, also every row of that head
    (every query block of every workgroup, whatever its place in the schedule)."""
    say(f"case {wl.name} causal={causal} (sampled rows, heads {heads}; every row of head {full_head})")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    o, l = host(*run_gpu(wl, t, causal))
    bm = fa.fa_varlen_block_sizes(wl.head_dim, dtype_code(fa, wl.dtype))[0]
    rows = sample_rows(wl, bm, np.random.default_rng(seed))
    ref_o, ref_l = attention_rows(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal, rows,
                                  heads)
    compare(o[rows][:, heads], l[heads][:, rows], ref_o, ref_l, TOL[wl.dtype], wl.name)
    assert not np.isnan(o[:wl.total_q]).any() and not np.isnan(l[:, :wl.total_q]).any()
    if full_head is not None:
        n = wl.total_q
        ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal,
                                     heads=[full_head])
        compare(o[:n, full_head], l[full_head, :n], ref_o[:n, full_head], ref_l[full_head, :n], TOL[wl.dtype],
                f"{wl.name} head {full_head}, all {n} rows")


@pytest.mark.parametrize("seqlen", SWEEP_SEQLENS)
@pytest.mark.parametrize("head_dim", SWEEP_HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_sampled(fa, seqlen, head_dim, causal):
    wl = workload_sweep(seqlen, head_dim)
    sampled_parity(fa, wl, causal, [0, wl.heads // 2, wl.heads - 1], seed=seqlen + head_dim,
                   full_head=wl.heads - 1 if seqlen >= 4096 else None)


def test_ragged64k_sampled(fa):
    wl = workload_ragged64k()
    sampled_parity(fa, wl, True, [0, 17, 31], seed=4, full_head=wl.heads - 1)


# ---------------------------------------------------------------- edge cases
EDGE = [
    ("empty_seqs", [0, 37, 0, 200, 0], [5, 0, 0, 300, 0]),
    ("single_tokens", [1, 1, 1, 2], [1, 3, 1, 1]),
    ("ragged_tails", [129, 63, 65, 191, 257], [129, 63, 65, 191, 257]),
    ("q_longer_than_k", [824, 300, 40], [724, 33, 1]),
    ("k_longer_than_q", [200, 5, 77], [300, 500, 130]),
    # key counts at and next to multiples of the 32-, 64- and 128-key tiles:
    # 1 to 8 tiles per item, so every preamble and end-of-loop branch of the
    # direct K/V loads (tiles still to load, tiles in flight) is taken
    ("tile_boundaries", [64, 128, 192, 256, 383, 384, 385, 512], [64, 128, 192, 256, 383, 384, 385, 512]),
]


@pytest.mark.parametrize("name,lq,lk", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("bf16", 96), ("bf16", 128), ("bf16", 256), ("f16", 64),
                                            ("f16", 96), ("f16", 128), ("f16", 256), ("f32", 64), ("f32", 96),
                                            ("f32", 128)])
def test_edge_cases(fa, name, lq, lk, dtype, head_dim):
    wl = workload_custom(f"{name}_{dtype}_d{head_dim}", lq, lk, 3, head_dim, dtype, seed=len(name) + head_dim)
    for causal in (False, True):
        full_parity(fa, wl, causal)


def test_many_short_sequences(fa):
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(0, 40, size=300)]
    wl = workload_custom("short300", lens, lens, 2, 128, "bf16", seed=77)
    for causal in (False, True):
        full_parity(fa, wl, causal)


@pytest.mark.parametrize("batch", [63, 64, 65])
def test_map_boundary(fa, batch):
    # fa_varlen_fwd rebuilds the work map inside the kernel up to 64 sequences
    # and launches the map kernel above; both must match the oracle and the
    # mapped entry point bit for bit (empty sequences at both ends included)
    rng = np.random.default_rng(100 + batch)
    lens = [int(x) for x in rng.integers(0, 600, size=batch)]
    lens[0] = lens[-1] = 0
    lens[batch // 2] = 0
    wl = workload_custom(f"map_boundary_b{batch}", lens, lens, 2, 128, "bf16", seed=90 + batch)
    data = draw_qkv(wl)
    t = to_device(data, wl)
    blk = fa.fa_varlen_tile_map(t["cu_q"], wl.max_seqlen_q, wl.head_dim, fa.FA_DTYPE_BF16)
    for causal in (False, True):
        say(f"case map boundary batch={batch} causal={causal}")
        o1, l1 = host(*run_gpu(wl, t, causal))
        o2, l2 = fa.fa_varlen_fwd_mapped(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q,
                                         wl.max_seqlen_k, blk, wl.scale, causal)
        torch.cuda.synchronize()
        o2, l2 = host(o2, l2)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        full_parity(fa, wl, causal)


def test_single_64k_sequence_sampled(fa):
    # one sequence of 65,536 tokens: the longest work items (1024 key tiles),
    # causal pairing of its 256 query blocks, and 64-bit offsets over the
    # whole K/V walk; 40 sampled rows per head (block edges included), both masks
    wl = workload_custom("long_64k_h2_d128", [65536], None, 2, 128, "bf16", seed=81)
    data = draw_qkv(wl)
    t = to_device(data, wl)
    rng = np.random.default_rng(81)
    rows = np.unique(np.concatenate([[0, 255, 256, 32767, 32768, 65279, 65280, 65535],
                                     rng.integers(0, 65536, size=32)])).astype(np.int64)
    for causal in (False, True):
        say(f"case {wl.name} causal={causal} ({len(rows)} sampled rows, both heads)")
        o, l = host(*run_gpu(wl, t, causal))
        ref_o, ref_l = attention_rows(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal, rows,
                                      [0, 1])
        compare(o[rows], l[:, rows], ref_o, ref_l, TOL["bf16"], wl.name)
        assert not np.isnan(o).any() and not np.isnan(l).any()


def test_70k_sequences(fa):
    # 70,000 sequences of 0-8 tokens (280k tokens): the map kernel's scan over
    # many chunks, ~70k work items per head, beyond the no-allocation entry
    # point's 65,535-sequence limit; every row against the oracle
    rng = np.random.default_rng(82)
    lens = [int(x) for x in rng.integers(0, 9, size=70000)]
    wl = workload_custom("many_70k_seqs_h2_d64", lens, None, 2, 64, "bf16", seed=82)
    for causal in (False, True):
        full_parity(fa, wl, causal)


def test_single_long_sequence_fp32(fa):
    wl = workload_custom("long_fp32", [2000], [2300], 2, 128, "f32", seed=78)
    for causal in (False, True):
        full_parity(fa, wl, causal)


def test_zero_queries_give_mean_of_visible_values(fa):
    """Q = 0: every visible key scores alike, so out is the mean of the visible V rows."""
    wl = workload_custom("q_zero", [300, 129], [280, 129], 2, 128, "bf16", seed=79)
    data = draw_qkv(wl)
    data["q"][:] = 0
    data["q_bits"][:] = 0
    t = to_device(data, wl)
    for causal in (False, True):
        say(f"case q_zero causal={causal}")
        o, l = host(*run_gpu(wl, t, causal))
        ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
        compare(o, l, ref_o, ref_l, TOL["bf16"], "q_zero")


# ---------------------------------------------------------------- buffers, determinism, mapped entry
def test_poisoned_and_guarded_buffers(fa):
    """Rows past cu_q[-1] and guard bands around out/lse stay untouched."""
    wl = workload_custom("guards", [100, 250], [100, 250], 2, 128, "bf16", seed=80)
    data = draw_qkv(wl)
    t = to_device(data, wl)
    extra, guard = 17, 64
    H, D, Tq = wl.heads, wl.head_dim, wl.total_q + extra
    q = torch.zeros((Tq, H, D), dtype=torch.bfloat16, device="cuda")
    q[:wl.total_q] = t["q"]
    big_o = torch.full((Tq + 2 * guard, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    big_l = torch.full((H * Tq + 2 * guard * 64,), float("nan"), dtype=torch.float32, device="cuda")
    out = big_o[guard:guard + Tq]
    lse = big_l[guard * 64:guard * 64 + H * Tq].view(H, Tq)
    for causal in (False, True):
        say(f"case guards causal={causal}")
        fa.fa_varlen_fwd(q, t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k, wl.scale,
                         causal, out=out, lse=lse)
        torch.cuda.synchronize()
        bo = big_o.float().cpu().numpy()
        bl = big_l.cpu().numpy()
        assert np.isnan(bo[:guard]).all() and np.isnan(bo[guard + Tq:]).all()
        assert np.isnan(bl[:guard * 64]).all() and np.isnan(bl[guard * 64 + H * Tq:]).all()
        o = bo[guard:guard + Tq]
        l = bl[guard * 64:guard * 64 + H * Tq].reshape(H, Tq)
        assert np.isnan(o[wl.total_q:]).all() and np.isnan(l[:, wl.total_q:]).all()
        ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
        compare(o[:wl.total_q], l[:, :wl.total_q], ref_o, ref_l, TOL["bf16"], "guards")


def test_deterministic_and_mapped_identical(fa):
    # queries longer than 1024 rows: fa_varlen_fwd takes the work items of
    # fa_varlen_block_sizes, as the mapped entry point does, so the two are
    # bit-identical; with 1024 rows or fewer (the 128-row items) they agree
    # to the parity bar and each is deterministic
    for wl in (workload_custom("mapped_long_d64", [1300, 200, 77], [1100, 300, 90], 6, 64, "bf16", seed=30),
               workload_custom("mapped_long_d128", [1025, 3], None, 4, 128, "f16", seed=31), workload_ragged_qk()):
        data = draw_qkv(wl)
        t = to_device(data, wl)
        code = fa.FA_DTYPE_BF16 if wl.dtype == "bf16" else fa.FA_DTYPE_F16
        blk = fa.fa_varlen_tile_map(t["cu_q"], wl.max_seqlen_q, wl.head_dim, code)
        for causal in (False, True):
            say(f"case determinism {wl.name} causal={causal}")
            o1, l1 = host(*run_gpu(wl, t, causal))
            o2, l2 = host(*run_gpu(wl, t, causal))
            o3, l3 = fa.fa_varlen_fwd_mapped(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q,
                                             wl.max_seqlen_k, blk, wl.scale, causal)
            torch.cuda.synchronize()
            o3, l3 = host(o3, l3)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
            if wl.max_seqlen_q > 1024:
                assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
            else:
                compare(o1, l1, o3, l3, TOL[wl.dtype], f"{wl.name}: short items vs mapped")


SHORT = [("short_d64_bf16", [1024, 1, 129, 700, 64, 1000, 0, 33], None, 64, "bf16"),
         ("short_d128_f16", [512, 1024, 255, 2, 97], [600, 1024, 100, 2, 300], 128, "f16"),
         ("short_d128_bf16_qk", [1000, 31, 400], [1500, 31, 200], 128, "bf16")]


@pytest.mark.parametrize("name,lq,lk,head_dim,dtype", SHORT, ids=[s[0] for s in SHORT])
@pytest.mark.parametrize("causal", [False, True])
def test_short_work_items(fa, name, lq, lk, head_dim, dtype, causal):
    """max_seqlen_q <= 1024 at head_dim 64/128: fa_varlen_fwd's 128-row work
    items (four wavefronts, 64- or 32-key tiles) against the oracle: ragged
    tails, empty and single-token sequences, Lq != Lk."""
    wl = workload_custom(name, lq, lk, 4, head_dim, dtype, seed=len(name) + head_dim, heads_k=2)
    say(f"case {wl.name} causal={causal}")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    o, l = host(*run_gpu(wl, t, causal))
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare(o[:wl.total_q], l[:, :wl.total_q], ref_o, ref_l, TOL[dtype], wl.name)


def test_check_cu_seqlens_flags(fa):
    def flags(cq, ck, tq, tk, mq, mk):
        a = torch.tensor(cq, dtype=torch.int32, device="cuda")
        b = torch.tensor(ck, dtype=torch.int32, device="cuda")
        return int(fa.fa_varlen_check_cu_seqlens(a, b, tq, tk, mq, mk).item())
    assert flags([0, 128, 300], [0, 128, 300], 300, 300, 172, 172) == 0
    assert flags([1, 128, 300], [0, 128, 300], 300, 300, 300, 300) == 1
    assert flags([0, 128, 100], [0, 128, 300], 300, 300, 300, 300) == 2
    assert flags([0, 128, 301], [0, 128, 300], 300, 300, 300, 300) == 4
    assert flags([0, 128, 300], [0, 128, 300], 300, 300, 171, 172) == 8
    assert flags([0, 128, 300], [0, 200, 100], 300, 300, 300, 300) == 32
    assert flags([0], [0], 0, 0, 0, 0) == 0


# ---------------------------------------------------------------- fp16 and shared key/value heads
def test_ragged_qk_f16(fa):
    base = workload_ragged_qk()
    wl = workload_custom("ragged_qk_h12_d64_f16", base.lengths_q, base.lengths_k, 12, 64, "f16", seed=5)
    for causal in (False, True):
        full_parity(fa, wl, causal)


def test_dense_f16_sampled(fa):
    wl = workload_custom("dense_8x2048_h16_d128_f16", [2048] * 8, None, 16, 128, "f16", seed=6)
    for causal in (False, True):
        sampled_parity(fa, wl, causal, [0, 9, 15], seed=6)


GQA = [(8, 1), (8, 2), (8, 4), (6, 3), (4, 4)]


@pytest.mark.parametrize("heads,heads_k", GQA, ids=[f"h{h}kv{k}" for h, k in GQA])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("bf16", 96), ("bf16", 128), ("bf16", 256), ("f16", 128),
                                            ("f32", 64), ("f32", 128)])
def test_shared_kv_heads(fa, heads, heads_k, dtype, head_dim):
    wl = workload_custom(f"gqa_h{heads}_kv{heads_k}_{dtype}_d{head_dim}", [300, 0, 129, 700], [280, 5, 200, 700],
                         heads, head_dim, dtype, seed=heads * 10 + heads_k, heads_k=heads_k)
    for causal in (False, True):
        full_parity(fa, wl, causal)


def test_ragged64k_gqa_sampled(fa):
    """The headline batch with 32 query heads sharing 8 key/value heads."""
    wl = workload_ragged64k_gqa()
    sampled_parity(fa, wl, True, [0, 3, 4, 31], seed=41)


# ---------------------------------------------------------------- head_dim 96
def test_ragged_qk_d96(fa):
    base = workload_ragged_qk()
    for dtype in ("bf16", "f32"):
        wl = workload_custom(f"ragged_qk_h12_d96_{dtype}", base.lengths_q, base.lengths_k, 12, 96, dtype, seed=7)
        for causal in (False, True):
            full_parity(fa, wl, causal)


def test_ragged64k_d96_sampled(fa):
    """The headline length mix (64k tokens, 32 heads) at head_dim 96."""
    base = workload_ragged64k()
    wl = workload_custom("ragged64k_h32_d96", base.lengths_q, None, 32, 96, "bf16", seed=8)
    for causal in (False, True):
        sampled_parity(fa, wl, causal, [0, 13, 31], seed=8)


# ---------------------------------------------------------------- head_dim 256
def test_ragged_qk_d256(fa):
    base = workload_ragged_qk()
    for dtype in ("bf16", "f16"):
        wl = workload_custom(f"ragged_qk_h12_d256_{dtype}", base.lengths_q, base.lengths_k, 12, 256, dtype, seed=9)
        for causal in (False, True):
            full_parity(fa, wl, causal)


def test_ragged64k_d256_sampled(fa):
    """The headline length mix (64k tokens) at head_dim 256 with 16 heads."""
    base = workload_ragged64k()
    wl = workload_custom("ragged64k_h16_d256", base.lengths_q, None, 16, 256, "bf16", seed=10)
    for causal in (False, True):
        sampled_parity(fa, wl, causal, [0, 7, 15], seed=10)


# ---------------------------------------------------------------- score spikes
SPIKE_CASES = [("bf16", 128), ("bf16", 64), ("bf16", 96), ("f16", 128), ("f16", 64), ("bf16", 256), ("f16", 256)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,head_dim", SPIKE_CASES, ids=[f"{d}_d{h}" for d, h in SPIKE_CASES])
def test_score_spikes_raise_reference(fa, causal, dtype, head_dim):
    """Keys multiplied by 16 (exact in bf16 and fp16) in the middle of long
    sequences give scores tens of log2 units above every earlier one, so the
    kernels must raise their softmax references and rescale the partial
    outputs in the middle of the key loop, not only in its first tiles."""
    spikes_case(fa, causal, dtype, head_dim, [2048, 1500, 700], [2048, 1700, 900])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f16", 64)], ids=["bf16_d128", "f16_d64"])
def test_score_spikes_short_items(fa, causal, dtype, head_dim):
    """The same with every query length at most 1024, where fa_varlen_fwd
    takes 128-row work items (four wavefronts, 32- or 64-key tiles)."""
    spikes_case(fa, causal, dtype, head_dim, [1024, 700, 301], [1024, 900, 501])


def spikes_case(fa, causal, dtype, head_dim, lq, lk):
    from fa_synth import bf16_rne_bits, f16_rne_bits
    wl = workload_custom(f"spikes_{dtype}_d{head_dim}_q{max(lq)}", lq, lk, 4, head_dim, dtype, seed=31)
    say(f"case {wl.name} causal={causal}")
    data = draw_qkv(wl)
    k = data["k"].copy()
    for b in range(wl.batch):
        k0, Lk = wl.cu_k[b], wl.cu_k[b + 1] - wl.cu_k[b]
        for frac in (0.37, 0.81):
            k[k0 + int(frac * Lk)] *= 16.0
    data["k"] = k
    data["k_bits"] = bf16_rne_bits(k) if dtype == "bf16" else f16_rne_bits(k)
    t = to_device(data, wl)
    o, l = host(*run_gpu(wl, t, causal))
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    n = wl.total_q
    compare(o[:n], l[:, :n], ref_o[:n], ref_l[:, :n], TOL[dtype], wl.name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f16", 64)])
def test_nan_inputs_stay_local(fa, causal, dtype, head_dim):
    """NaN propagation (the pages leave it open; the reading here is the
    oracle's row-wise definition): a NaN anywhere in a query row makes that
    (row, head)'s out and lse NaN and nothing else; a NaN in a key makes NaN
    exactly the rows that see that key, under the causal mask too.  Every
    other row matches the oracle at the usual bar.  (NaN in V is not covered:
    a product of a zero probability and a NaN value is NaN in any matrix
    product, so which rows it reaches depends on how keys are blocked.)"""
    from fa_synth import bf16_rne_bits, f16_rne_bits
    wl = workload_custom(f"nan_{dtype}_d{head_dim}", [300, 200, 64], [300, 250, 64], 4, head_dim, dtype, seed=34)
    say(f"case {wl.name} causal={causal}")
    data = draw_qkv(wl)
    q, k = data["q"].copy(), data["k"].copy()
    q[17, 1, :] = np.nan                  # a whole query row, sequence 0, head 1
    q[300 + 50, 2, 5] = np.nan            # one element of a query row, sequence 1, head 2
    k[500 + 40, 0, 3] = np.nan            # one element of key 40 of sequence 2 (key/value head 0)
    data["q"], data["k"] = q, k
    rnd = bf16_rne_bits if dtype == "bf16" else f16_rne_bits
    data["q_bits"], data["k_bits"] = rnd(q), rnd(k)
    t = to_device(data, wl)
    o, l = host(*run_gpu(wl, t, causal))
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    n = wl.total_q
    o, l, ref_o, ref_l = o[:n], l[:, :n], ref_o[:n], ref_l[:, :n]
    bad = np.isnan(ref_l)                 # (head, row) pairs the definition makes NaN
    assert bad.sum() > 2, "the planted NaNs must reach the key's rows too"
    for h in range(wl.heads):
        assert np.array_equal(np.isnan(l[h]), bad[h]), f"head {h}: NaN lse pattern differs from the oracle"
        assert np.isnan(o[:, h][bad[h]]).all(), f"head {h}: out of a NaN row must be NaN"
    o_ok = np.where(bad.T[:, :, None], 0.0, o)
    r_ok = np.where(bad.T[:, :, None], 0.0, ref_o)
    l_ok = np.where(bad, 0.0, l)
    lr_ok = np.where(bad, 0.0, ref_l)
    compare(o_ok, l_ok, r_ok, lr_ok, TOL[dtype], wl.name)
