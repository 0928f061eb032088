"""GPU parity of attention against a key/value cache (fa_varlen_fwd_kvcache)
through the C ABI, against oracle.kvcache.

Bar: as the forward pass (the same arithmetic: 16-bit MFMA products, fp32
online softmax, P rounded to the input type): max-abs 2e-2 for bf16, 5e-3
for fp16 and 1e-5 for fp32 (fp32 MFMA products, P kept in fp32) on out and
lse; rows with no visible key give out = 0 and lse = -inf exactly.  Cases: plain and paged caches (pages of 16 and 256 rows), left
padding, empty and single-key sequences, key lengths around the 32-key tile,
one and several query rows per sequence (up to several 32-row tiles of
query-head x row), causal and not, MHA/GQA/MQA, explicit split counts
including more splits than tiles, fp16, fp32, and the bench's decode batch at
full size, and head_dim 64, 96 and 256 besides 128.
"""
import numpy as np
import pytest

from fa_synth import draw_kvcache, workload_decode, workload_decode_bench
from oracle import attention_kvcache
from tests._gpu_util import TOL, compare, say

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def fa():
    import variable_length_flashattention_cu_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback exists
    return m


def run_case(fa, wl, causal, num_splits=0):
    say(f"case {wl.name} causal={causal} splits={num_splits}")
    data = draw_kvcache(wl)
    names = ("q", "k_cache", "v_cache")
    if wl.dtype == "f32":
        dev = {n: torch.from_numpy(data[n]).cuda() for n in names}
    else:
        tt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        dev = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).cuda().view(tt) for n in names}
    cu_q = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    sk = torch.tensor(wl.seqlens_k, dtype=torch.int32, device="cuda")
    lp = None if wl.leftpad is None else torch.tensor(wl.leftpad, dtype=torch.int32, device="cuda")
    bt = None if not wl.paged else torch.from_numpy(data["block_table"]).cuda()
    out, lse = fa.fa_varlen_fwd_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], cu_q, sk, wl.max_seqlen_q,
                                        wl.max_seqlen_k, wl.scale, causal, leftpad_k=lp, block_table=bt,
                                        num_splits=num_splits)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    ref_o, ref_l = attention_kvcache(data["q"], data["k_cache"], data["v_cache"], wl.cu_q, wl.seqlens_k, wl.scale,
                                     causal, leftpad_k=wl.leftpad, block_table=data.get("block_table"),
                                     page_size=wl.cache_rows if wl.paged else None)
    n = wl.total_q
    compare(o[:n], l[:, :n], ref_o[:n], ref_l[:, :n], TOL[wl.dtype], wl.name)


SEQLENS = [0, 1, 31, 32, 33, 500, 77]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads,heads_k", [(8, 2), (4, 4), (8, 1)], ids=["gqa", "mha", "mqa"])
def test_decode_plain(fa, causal, heads, heads_k):
    wl = workload_decode(f"dec_plain_h{heads}kv{heads_k}", [1] * len(SEQLENS), SEQLENS, heads, heads_k, 128, "bf16",
                         seed=31 + heads_k, cache_rows=520)
    run_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_leftpad(fa, causal):
    wl = workload_decode("dec_leftpad", [1, 2, 1, 3], [40, 300, 5, 129], 8, 2, 128, "bf16", seed=32, cache_rows=300,
                         leftpad=[7, 100, 5, 0])
    run_case(fa, wl, causal)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("head_dim", [64, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_head_dims(fa, head_dim, dtype, causal):
    # every head_dim the decode kernels take besides the 128 of the other
    # cases: paged cache with left padding, GQA, several query rows per
    # sequence, an empty and a single-key sequence, tile-edge key lengths
    wl = workload_decode(f"dec_d{head_dim}_{dtype}", [1, 3, 1, 2, 1], [0, 300, 1, 64, 97], 6, 2, head_dim, dtype,
                         seed=40 + head_dim, cache_rows=32, leftpad=[0, 17, 0, 3, 0], paged=True)
    run_case(fa, wl, causal, num_splits=3)


@pytest.mark.parametrize("page", [16, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged(fa, page, causal):
    wl = workload_decode(f"dec_paged{page}", [1, 1, 2, 1, 4], [700, 1, 300, 0, 257], 8, 2, 128, "bf16", seed=33,
                         cache_rows=page, leftpad=[10, 0, 44, 0, 3], paged=True)
    run_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_many_rows(fa, causal):
    # 8 query heads per key/value head: 4 rows -> one 32-row tile; 40 rows -> 10 tiles
    wl = workload_decode("dec_rows", [4, 40, 1, 0], [200, 333, 64, 50], 16, 2, 128, "bf16", seed=34, cache_rows=333)
    run_case(fa, wl, causal)


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_decode_explicit_splits(fa, splits):
    wl = workload_decode("dec_splits", [1, 1, 2], [1000, 40, 513], 8, 2, 128, "bf16", seed=35, cache_rows=1024,
                         leftpad=[0, 8, 1])
    run_case(fa, wl, True, num_splits=splits)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_f16_d64(fa, causal):
    wl = workload_decode("dec_f16_d64", [1, 3, 1], [90, 257, 33], 8, 4, 64, "f16", seed=36, cache_rows=64,
                         leftpad=[0, 2, 1], paged=True)
    run_case(fa, wl, causal)


@pytest.mark.parametrize("head_dim", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_f32(fa, head_dim, causal):
    # fp32 caches (fp32 MFMA kernel): paged with left padding, GQA, several
    # query rows per sequence, an empty and a single-key sequence, key lengths
    # around the 32-key tile, 3 splits
    wl = workload_decode(f"dec_f32_d{head_dim}", [1, 3, 1, 2, 1, 5], [0, 300, 1, 64, 97, 33], 6, 2, head_dim, "f32",
                         seed=50 + head_dim, cache_rows=32, leftpad=[0, 17, 0, 3, 0, 1], paged=True)
    run_case(fa, wl, causal, num_splits=3)


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_f32_plain(fa, splits):
    # fp32 without a block table, MQA, automatic and single split
    wl = workload_decode("dec_f32_plain", [1, 2, 1, 1], [700, 129, 32, 0], 8, 1, 128, "f32", seed=58,
                         cache_rows=704)
    run_case(fa, wl, True, num_splits=splits)


def test_decode_bench_batch(fa):
    """The bench's decode batch at full size (32 sequences, 1k-16k cached keys, paged)."""
    run_case(fa, workload_decode_bench(), True)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_nan_inputs_stay_local(fa, causal):
    """NaN propagation through the split key ranges and their merge: a NaN in
    a query row makes that (row, head) NaN, a NaN in a cached key makes NaN
    exactly the rows that see it (the oracle's row-wise definition); every
    other row matches at the usual bar."""
    from fa_synth import bf16_rne_bits
    wl = workload_decode("dec_nan", [1, 3, 1], [400, 300, 90], 8, 2, 128, "bf16", seed=37, cache_rows=32,
                         leftpad=[0, 5, 0], paged=True)
    say(f"case {wl.name} causal={causal}")
    data = draw_kvcache(wl)
    q, kc = data["q"].copy(), data["k_cache"].copy()
    q[2, 3, :] = np.nan                                   # sequence 1, its second row, head 3
    tbl = data["block_table"]
    blk, row = int(tbl[2, 50 // 32]), 50 % 32             # sequence 2, cache position 50, key/value head 1
    kc[blk, row, 1, 7] = np.nan
    data["q"], data["k_cache"] = q, kc
    data["q_bits"], data["k_cache_bits"] = bf16_rne_bits(q).reshape(q.shape), bf16_rne_bits(kc).reshape(kc.shape)
    dev = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
           for n in ("q", "k_cache", "v_cache")}
    cu_q = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    sk = torch.tensor(wl.seqlens_k, dtype=torch.int32, device="cuda")
    lp = torch.tensor(wl.leftpad, dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(tbl).cuda()
    out, lse = fa.fa_varlen_fwd_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], cu_q, sk, wl.max_seqlen_q,
                                        wl.max_seqlen_k, wl.scale, causal, leftpad_k=lp, block_table=bt,
                                        num_splits=3)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    ref_o, ref_l = attention_kvcache(data["q"], data["k_cache"], data["v_cache"], wl.cu_q, wl.seqlens_k, wl.scale,
                                     causal, leftpad_k=wl.leftpad, block_table=tbl, page_size=wl.cache_rows)
    bad = np.isnan(ref_l)
    assert bad.sum() >= 2
    assert np.array_equal(np.isnan(l), bad), "NaN lse pattern differs from the oracle"
    assert np.isnan(o.transpose(1, 0, 2)[bad]).all(), "out of a NaN row must be NaN"
    keep = ~bad.T[:, :, None]
    compare(np.where(keep, o, 0.0), np.where(bad, 0.0, l), np.where(keep, ref_o, 0.0), np.where(bad, 0.0, ref_l),
            TOL["bf16"], wl.name)
