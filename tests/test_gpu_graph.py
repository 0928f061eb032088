"""Entry points under HIP graph capture (they allocate nothing when the
caller passes every buffer, and issue no memset).

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


def test_backward_replays_in_a_graph(fa):
    """fa_varlen_bwd with caller-owned outputs and workspace (the library then
    allocates nothing): the prep, main and dq kernels captured and replayed.
    dk and dv are deterministic and must match an eager call bit for bit; dq
    is summed with float atomics, so it is compared within a bf16 ulp."""
    from fa_synth import draw_dout
    wl = workload_custom("graph_bwd_h4kv2_d128", [300, 0, 129, 700], [280, 5, 129, 900], 4, 128, "bf16",
                         seed=63, heads_k=2)
    say(f"case {wl.name}")
    data = draw_qkv(wl)
    t = to_device(data, wl)
    dout = torch.from_numpy(draw_dout(wl)["dout_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    out, lse = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                wl.scale, True)
    ws = torch.empty(fa.fa_varlen_bwd_workspace_size(wl.batch, wl.total_q, wl.heads, wl.head_dim),
                     dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])]

    def call(g):
        fa.fa_varlen_bwd(t["q"], t["k"], t["v"], out, dout, lse, t["cu_q"], t["cu_k"], wl.max_seqlen_q,
                         wl.max_seqlen_k, wl.scale, True, dq=g[0], dk=g[1], dv=g[2], workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(grads)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(grads)
    torch.cuda.synchronize()
    eager = [torch.empty_like(x) for x in grads]
    for rep in range(3):
        for x in grads:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(grads[1], eager[1]) and torch.equal(grads[2], eager[2]), f"replay {rep}: dk/dv differ"
        dq, dq_e = grads[0].float(), eager[0].float()
        assert not torch.isnan(dq).any()
        assert float((dq - dq_e).abs().max()) <= 2.0 ** -7 * float(dq_e.abs().max()), f"replay {rep}: dq differs"
        say(f"  replay {rep}: dk, dv identical, dq within a bf16 ulp of the eager call")


def test_kvcache_replays_in_a_graph(fa):
    """fa_varlen_fwd_kvcache with caller-owned out, lse and workspace: the
    split pass and the combine kernel captured and replayed; the cache is
    changed in place between replays.  Every replay equals an eager call."""
    from fa_synth import draw_kvcache, workload_decode
    wl = workload_decode("graph_kv_h8kv2_d128", [1, 2, 1, 1], [300, 41, 0, 700], 8, 2, 128, "bf16", seed=64,
                         cache_rows=64, leftpad=[3, 0, 0, 17], paged=True)
    say(f"case {wl.name}")
    data = draw_kvcache(wl)
    dev = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
           for n in ("q", "k_cache", "v_cache")}
    cu_q = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    sk = torch.tensor(wl.seqlens_k, dtype=torch.int32, device="cuda")
    lp = torch.tensor(wl.leftpad, dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(data["block_table"]).cuda()
    ws = torch.empty(fa.fa_varlen_kvcache_workspace_size(wl.total_q, wl.heads, wl.head_dim, 0), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((wl.heads, wl.total_q), dtype=torch.float32, device="cuda")

    def call(o, l):
        fa.fa_varlen_fwd_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], cu_q, sk, wl.max_seqlen_q,
                                 wl.max_seqlen_k, wl.scale, True, leftpad_k=lp, block_table=bt, out=o, lse=l,
                                 workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(out, lse)
    torch.cuda.synchronize()
    eo, el = torch.empty_like(out), torch.empty_like(lse)
    for rep in range(3):
        if rep == 1:
            dev["v_cache"].mul_(-2.0)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay {rep}: differs from the eager call"
        say(f"  replay {rep}: identical to the eager call")
