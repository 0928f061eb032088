"""Seeded random shapes through the HIP path against the oracle, every row.

The shapes are drawn once from fixed seeds, so every run checks the same
cases.  They mix empty and single-token sequences, lengths on and off the
tile edges, Lq != Lk, shared key/value heads, every head_dim and dtype each
entry point takes, both mask modes, and batch sizes on both sides of 64
sequences (where fa_varlen_fwd switches from rebuilding the work map in every
wavefront to the map kernel).  Bars: the forward and cache passes as
tests/_gpu_util.TOL (max-abs on out and finite lse, -inf exactly), the
backward as tests/test_gpu_bwd.py (RMS and max relative to the reference,
exact zeros).
"""
import math

import numpy as np
import pytest

from fa_synth import draw_kvcache, draw_qkv, workload_custom, workload_decode
from oracle import attention_fwd, attention_kvcache
from tests._gpu_util import TOL, compare, say, to_device
from tests.test_gpu_bwd import compare_grads, exact_zeros, run_fwd_bwd

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def fa():
    import variable_length_flashattention_cu_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback exists
    return m


def _length(rng, hi):
    """0 and 1 now and then, a tile edge (+-1) now and then, else log-uniform in [2, hi]."""
    u = rng.random()
    if u < 0.08:
        return 0
    if u < 0.16:
        return 1
    if u < 0.36:
        edge = int(rng.choice([32, 64, 128, 256, 512]))
        return max(0, min(hi, edge + int(rng.integers(-1, 2))))
    return int(round(math.exp(rng.uniform(math.log(2), math.log(hi)))))


def _heads(rng, max_h):
    h = int(rng.choice([x for x in (1, 2, 3, 4, 6, 8) if x <= max_h]))
    hk = int(rng.choice([d for d in range(1, h + 1) if h % d == 0]))
    return h, hk


def _dtype_dim(rng):
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.5, 0.3, 0.2]))
    dims = (64, 96, 128) if dtype == "f32" else (64, 96, 128, 256)
    return dtype, int(rng.choice(dims))


def _fwd_cases(n=32, seed=7100):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        batch = int(rng.choice([1, 2, 5, 17, 63, 64, 65, 90]))
        hi = max(2, 6000 // batch)
        lq = [_length(rng, min(hi, 1500)) for _ in range(batch)]
        lk = None if rng.random() < 0.6 else [_length(rng, min(hi, 1500)) for _ in range(batch)]
        h, hk = _heads(rng, 8 if sum(lq) < 3000 else 4)
        dtype, d = _dtype_dim(rng)
        causal = bool(rng.random() < 0.5)
        cases.append((f"fwd{i}_b{batch}_h{h}kv{hk}_d{d}_{dtype}", lq, lk, h, hk, d, dtype, causal, seed + i))
    return cases


def _bwd_cases(n=16, seed=7200):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        batch = int(rng.choice([1, 3, 6, 12]))
        lq = [_length(rng, 700) for _ in range(batch)]
        lk = None if rng.random() < 0.6 else [_length(rng, 700) for _ in range(batch)]
        h, hk = _heads(rng, 4)
        dtype, d = _dtype_dim(rng)
        causal = bool(rng.random() < 0.5)
        cases.append((f"bwd{i}_b{batch}_h{h}kv{hk}_d{d}_{dtype}", lq, lk, h, hk, d, dtype, causal, seed + i))
    return cases


def _kv_cases(n=16, seed=7300):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        batch = int(rng.choice([1, 4, 9, 20]))
        seqlens = [_length(rng, 1200) for _ in range(batch)]
        rows = [int(rng.choice([0, 1, 1, 1, 2, 5])) for _ in range(batch)]
        leftpad = None if rng.random() < 0.5 else [int(rng.integers(0, s + 1)) for s in seqlens]
        h, hk = _heads(rng, 8)
        dtype, d = _dtype_dim(rng)
        paged = bool(rng.random() < 0.5)
        cache_rows = int(rng.choice([16, 64, 256])) if paged else max(1, max(seqlens))
        causal = bool(rng.random() < 0.5)
        splits = int(rng.choice([0, 0, 1, 3, 7]))
        cases.append((f"kv{i}_b{batch}_h{h}kv{hk}_d{d}_{dtype}", rows, seqlens, leftpad, h, hk, d, dtype, paged,
                       cache_rows, causal, splits, seed + i))
    return cases


FWD = _fwd_cases()
BWD = _bwd_cases()
KV = _kv_cases()


@pytest.mark.parametrize("case", FWD, ids=[c[0] for c in FWD])
def test_random_forward(fa, case):
    name, lq, lk, h, hk, d, dtype, causal, seed = case
    wl = workload_custom(name, lq, lk, h, d, dtype, seed=seed, heads_k=hk)
    say(f"case {name} causal={causal} lq={lq} lk={lk}")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    out, lse = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                wl.scale, causal)
    torch.cuda.synchronize()
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[dtype], name)


@pytest.mark.parametrize("case", BWD, ids=[c[0] for c in BWD])
def test_random_backward(fa, case):
    from oracle import attention_bwd
    name, lq, lk, h, hk, d, dtype, causal, seed = case
    wl = workload_custom(name, lq, lk, h, d, dtype, seed=seed, heads_k=hk)
    say(f"case {name} causal={causal} lq={lq} lk={lk}")
    data, g, got = run_fwd_bwd(fa, wl, causal)
    ref = attention_bwd(data["q"], data["k"], data["v"], g["dout"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare_grads(got, ref, dtype, name)
    exact_zeros(wl, causal, got)


@pytest.mark.parametrize("case", KV, ids=[c[0] for c in KV])
def test_random_kvcache(fa, case):
    name, rows, seqlens, leftpad, h, hk, d, dtype, paged, cache_rows, causal, splits, seed = case
    wl = workload_decode(name, rows, seqlens, h, hk, d, dtype, seed=seed, cache_rows=cache_rows, leftpad=leftpad,
                         paged=paged)
    say(f"case {name} causal={causal} rows={rows} seqlens={seqlens} leftpad={leftpad} paged={paged} "
        f"cache_rows={cache_rows} splits={splits}")
    data = draw_kvcache(wl)
    names = ("q", "k_cache", "v_cache")
    if dtype == "f32":
        dev = {n: torch.from_numpy(data[n]).cuda() for n in names}
    else:
        tt = torch.bfloat16 if dtype == "bf16" else torch.float16
        dev = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).cuda().view(tt) for n in names}
    cu_q = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    sk = torch.tensor(wl.seqlens_k, dtype=torch.int32, device="cuda")
    lp = None if wl.leftpad is None else torch.tensor(wl.leftpad, dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(data["block_table"]).cuda() if paged else None
    out, lse = fa.fa_varlen_fwd_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], cu_q, sk, wl.max_seqlen_q,
                                        wl.max_seqlen_k, wl.scale, causal, leftpad_k=lp, block_table=bt,
                                        num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = attention_kvcache(data["q"], data["k_cache"], data["v_cache"], wl.cu_q, wl.seqlens_k, wl.scale,
                                     causal, leftpad_k=wl.leftpad, block_table=data.get("block_table"),
                                     page_size=cache_rows if paged else None)
    n = wl.total_q
    compare(out.float().cpu().numpy()[:n], lse.cpu().numpy()[:, :n], ref_o[:n], ref_l[:, :n], TOL[dtype], name)
