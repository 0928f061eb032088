"""fa_varlen_fwd_noalloc through the C ABI: the same results as fa_varlen_fwd
(bit for bit: the same kernels read the same map), within the oracle bar, on
two calls in a row -- the second on a smaller batch, so that it reads a map
the first call left behind in the static scratch and must overwrite."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from fa_synth import draw_qkv, workload_custom  # noqa: E402
from oracle import attention_fwd  # noqa: E402
from tests._gpu_util import TOL, compare, host, say, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import variable_length_flashattention_cu_amd as fa
    fa.load_library()
    return fa


def run_pair(fa, wl, causal):
    data = draw_qkv(wl)
    t = to_device(data, wl)
    out_a, lse_a = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                    wl.scale, causal)
    # caller-allocated outputs, poisoned so that an unwritten row shows
    out_b = torch.full_like(t["q"], float("nan"))
    lse_b = torch.full((wl.heads, wl.total_q), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_varlen_fwd_noalloc(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                             out_b, lse_b, wl.scale, causal)
    torch.cuda.synchronize()
    oa, la = host(out_a, lse_a)
    ob, lb = host(out_b, lse_b)
    assert np.array_equal(oa, ob, equal_nan=True) and np.array_equal(la, lb, equal_nan=True), wl.name
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare(ob, lb, ref_o, ref_l, TOL[wl.dtype], f"{wl.name} noalloc")


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_fwd_twice_second_smaller(fa, causal):
    big = workload_custom("noalloc_big", [700, 1, 0, 300, 513, 256, 90], [650, 5, 3, 300, 600, 256, 128], 4, 128,
                          "bf16", seed=21, heads_k=2)
    small = workload_custom("noalloc_small", [129, 64], [200, 64], 4, 128, "bf16", seed=22, heads_k=2)
    for wl in (big, small):
        say(f"case noalloc {wl.name} causal={causal} batch={wl.batch}")
        run_pair(fa, wl, causal)


def test_noalloc_other_dtypes(fa):
    for wl, causal in ((workload_custom("noalloc_f16_d64", [300, 33], None, 2, 64, "f16", seed=23), True),
                       (workload_custom("noalloc_f32_d96", [130, 70], [100, 90], 2, 96, "f32", seed=24), False)):
        say(f"case noalloc {wl.name} causal={causal}")
        run_pair(fa, wl, causal)
