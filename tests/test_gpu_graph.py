"""The allocation-free forward entry point under HIP graph capture.

fa_varlen_fwd_noalloc is meant for callers that cannot allocate, code under
graph capture among them.  Its launches (the work-item map into the library's
static array, then the attention kernel) are captured once into a graph and
replayed several times, with eager work between the replays: outputs cleared
to NaN, and the query tensor changed in place.  Every replay must equal an
eager call on the same inputs bit for bit, and the first one the oracle.
"""
import numpy as np
import pytest

from fa_synth import draw_qkv, workload_custom
from oracle import attention_fwd
from tests._gpu_util import TOL, compare, say, to_device

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def fa():
    import variable_length_flashattention_cu_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback exists
    return m


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("many", [False, True], ids=["5seqs", "80seqs"])
def test_noalloc_forward_replays_in_a_graph(fa, causal, many):
    # each capture holds two launches: the map kernel, writing the library's
    # static array, and the attention kernel reading it
    if many:
        rng = np.random.default_rng(62)
        lq = [int(x) for x in rng.integers(0, 200, size=80)]
        lk = [int(x) for x in rng.integers(0, 200, size=80)]
    else:
        lq, lk = [300, 0, 129, 700, 1], [280, 5, 129, 900, 1]
    wl = workload_custom(f"graph_b{len(lq)}_h4kv2_d128", lq, lk, 4, 128, "bf16", seed=61, heads_k=2)
    say(f"case {wl.name} causal={causal}")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    out = torch.empty_like(t["q"])
    lse = torch.empty((wl.heads, wl.total_q), dtype=torch.float32, device="cuda")

    def call(o, l):
        fa.fa_varlen_fwd_noalloc(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                 o, l, wl.scale, causal)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, lse)  # first call outside the capture: the static map's address is resolved here
    torch.cuda.synchronize()
    n = wl.total_q
    ref_o, ref_l = attention_fwd(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare(out.float().cpu().numpy()[:n], lse.cpu().numpy()[:, :n], ref_o[:n], ref_l[:, :n], TOL["bf16"],
            "eager")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(out, lse)
    torch.cuda.synchronize()

    eager_o, eager_l = torch.empty_like(out), torch.empty_like(lse)
    for rep in range(4):
        if rep == 2:
            t["q"].mul_(-0.5)  # new inputs behind the same pointers
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(eager_o, eager_l)
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o), f"replay {rep}: out differs from the eager call"
        assert torch.equal(lse, eager_l), f"replay {rep}: lse differs from the eager call"
        say(f"  replay {rep}: identical to the eager call")
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
