"""GPU parity of the backward pass: fa_varlen_fwd then fa_varlen_bwd through the
C ABI, against the float64 gradients of oracle.attention_grad.

Bar for 16-bit inputs (derived from the arithmetic; u = 2^-9 for bf16,
2^-11 for fp16, the unit roundoff of the operand type): every gradient element is a sum of
products in which one factor was rounded to the operand type (P before
dV = P^T dO, dS before dK and dQ, the forward's 16-bit out inside
D_i = rowsum(dO * out)), with float32 accumulation.  The roundings are
independent, so the error of a sum grows like its value and the relative
RMS error of each gradient tensor is a small multiple of u; single elements
can reach a few times that.  Checked, per tensor over the rows of all
sequences:
    RMS(err) <= 8u * RMS(ref)      max|err| <= 32u * max|ref|
For fp32 inputs nothing is rounded to a narrower type: the error comes from
float32 accumulation of sums of up to a few thousand terms (random-sign
roundings: relative RMS error of order sqrt(n) u, u = 2^-24, sqrt(2048) < 46),
from the forward's float32 out and lse (D_i and P inherit their relative
errors) and from the hardware exp2/log2 (a few ulp each); checked as
    RMS(err) <= 256u * RMS(ref)    max|err| <= 2048u * max|ref|
No NaN anywhere; rows that see no key have dq = 0 and keys no query sees
have dk = dv = 0 exactly.

Cases: ragged batches with empty sequences, single tokens, Lq != Lk under the
causal mask, tails of every size; head_dim 64, 96, 128 and 256; shared
key/value heads; fp16 and fp32; the bench's 64k-token length mix at full size with the oracle on a subset of
sequences and heads.
"""
import numpy as np
import pytest

from fa_synth import draw_dout, draw_qkv, workload_custom, workload_ragged64k, workload_ragged_qk
from oracle import attention_bwd, visible_mask
from tests._gpu_util import say, to_device

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U = {"bf16": 2.0 ** -9, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
# (RMS, max) multiples of u: see the module docstring
BAR = {"bf16": (8, 32), "f16": (8, 32), "f32": (256, 2048)}


@pytest.fixture(scope="module")
def fa():
    import variable_length_flashattention_cu_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback exists
    return m


def run_fwd_bwd(fa, wl, causal, workspace=None):
    data = draw_qkv(wl)
    g = draw_dout(wl)
    t = to_device(data, wl)
    if wl.dtype == "f32":
        dout = torch.from_numpy(g["dout"]).to("cuda")
    else:
        tt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        dout = torch.from_numpy(g["dout_bits"].view(np.int16)).to("cuda").view(tt)
    out, lse = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q,
                                wl.max_seqlen_k, wl.scale, causal)
    dq, dk, dv = fa.fa_varlen_bwd(t["q"], t["k"], t["v"], out, dout, lse, t["cu_q"], t["cu_k"],
                                  wl.max_seqlen_q, wl.max_seqlen_k, wl.scale, causal, workspace=workspace)
    torch.cuda.synchronize()
    host = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    return data, g, host


def compare_grads(got, ref, dtype, what):
    u = U[dtype]
    k_rms, k_max = BAR[dtype]
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        rows = ~np.isnan(r).any(axis=(1, 2))          # rows the oracle computed
        x, r = x[rows].astype(np.float64), r[rows]
        assert not np.isnan(x).any(), f"{what} {name}: NaN"
        if r.size == 0:
            continue
        err = np.abs(x - r)
        rms_ref = float(np.sqrt(np.mean(r * r)))
        rms_err = float(np.sqrt(np.mean(err * err)))
        max_ref = float(np.abs(r).max())
        max_err = float(err.max())
        say(f"  {what} {name}: rms err/ref {rms_err / max(rms_ref, 1e-30):.2e} "
            f"max err/ref {max_err / max(max_ref, 1e-30):.2e} (bounds {k_rms * u:.1e}, {k_max * u:.1e})")
        assert rms_err <= k_rms * u * rms_ref + 1e-30, f"{what} {name}: rms error {rms_err} vs {rms_ref}"
        assert max_err <= k_max * u * max_ref + 1e-30, f"{what} {name}: max error {max_err} vs {max_ref}"


def exact_zeros(wl, causal, got):
    """Rows with no visible key: dq == 0; keys nobody sees: dk == dv == 0."""
    dq, dk, dv = got
    for b in range(wl.batch):
        q0, q1, k0, k1 = wl.cu_q[b], wl.cu_q[b + 1], wl.cu_k[b], wl.cu_k[b + 1]
        vis = visible_mask(q1 - q0, k1 - k0, causal)
        none = ~vis.any(axis=1)
        assert np.all(dq[q0:q1][none] == 0), f"sequence {b}: dq of rows that see no key"
        unseen = ~vis.any(axis=0)
        assert np.all(dk[k0:k1][unseen] == 0) and np.all(dv[k0:k1][unseen] == 0), f"sequence {b}: unseen keys"


def full_case(fa, wl, causal):
    say(f"case {wl.name} causal={causal} dtype={wl.dtype}")
    data, g, got = run_fwd_bwd(fa, wl, causal)
    ref = attention_bwd(data["q"], data["k"], data["v"], g["dout"], wl.cu_q, wl.cu_k, wl.scale, causal)
    compare_grads(got, ref, wl.dtype, wl.name)
    exact_zeros(wl, causal, got)


EDGE = [
    ("empty_seqs", [0, 37, 0, 200, 0], [5, 0, 0, 300, 0]),
    ("single_tokens", [1, 1, 1, 2], [1, 3, 1, 1]),
    ("ragged_tails", [129, 63, 65, 191, 257], [129, 63, 65, 191, 257]),
    ("wide_block_tails", [255, 256, 513, 40], [255, 256, 513, 600]),
    ("q_longer_than_k", [824, 300, 40], [724, 33, 1]),
    ("k_longer_than_q", [200, 5, 77], [300, 500, 130]),
]


@pytest.mark.parametrize("name,lq,lk", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 64), ("bf16", 96), ("bf16", 128), ("f16", 64), ("f16", 96),
                                             ("f16", 128), ("bf16", 256), ("f16", 256), ("f32", 64), ("f32", 96),
                                             ("f32", 128)])
def test_bwd_edge_cases(fa, name, lq, lk, dtype, head_dim):
    wl = workload_custom(f"bwd_{name}_{dtype}_d{head_dim}", lq, lk, 3, head_dim, dtype, seed=len(name) + head_dim)
    for causal in (False, True):
        full_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_qk(fa, causal):
    base = workload_ragged_qk()
    wl = workload_custom("bwd_ragged_qk_h12_d64", base.lengths_q, base.lengths_k, 12, 64, "bf16", seed=21)
    full_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_d96(fa, causal):
    # head_dim 96: rows in 128-element LDS slots, dQ tiles on 6 of the 8 wavefronts
    wl = workload_custom("bwd_dense_3x1024_h4_d96", [1024] * 3, None, 4, 96, "f16", seed=23)
    full_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_d128(fa, causal):
    wl = workload_custom("bwd_dense_4x1024_h4_d128", [1024] * 4, None, 4, 128, "bf16", seed=22)
    full_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_d256(fa, causal):
    # head_dim 256: the 64-key workgroup (K and V of a key in registers, 16x16 MFMAs)
    wl = workload_custom("bwd_dense_2x1024_h4_d256", [1024] * 2, None, 4, 256, "bf16", seed=25)
    full_case(fa, wl, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_f32(fa, causal):
    wl = workload_custom("bwd_dense_2x1024_h4_d128_f32", [1024] * 2, None, 4, 128, "f32", seed=26)
    full_case(fa, wl, causal)


GQA = [(8, 1), (8, 2), (6, 3)]


@pytest.mark.parametrize("heads,heads_k", GQA, ids=[f"h{h}kv{k}" for h, k in GQA])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f16", 64), ("bf16", 96), ("f16", 256), ("f32", 96)])
def test_bwd_shared_kv_heads(fa, heads, heads_k, dtype, head_dim):
    wl = workload_custom(f"bwd_gqa_h{heads}_kv{heads_k}_{dtype}_d{head_dim}", [300, 0, 129, 700],
                         [280, 5, 200, 700], heads, head_dim, dtype, seed=heads * 10 + heads_k, heads_k=heads_k)
    for causal in (False, True):
        full_case(fa, wl, causal)


def test_bwd_ragged64k_sampled(fa):
    """The 64k-token length mix (32 heads, d=128, causal) at full size; the
    oracle covers four sequences of moderate length and two query heads."""
    base = workload_ragged64k()
    wl = workload_custom("bwd_ragged64k_h32_d128", base.lengths_q, None, 32, 128, "bf16", seed=23)
    say(f"case {wl.name} causal=True (sampled sequences and heads)")
    data, g, got = run_fwd_bwd(fa, wl, True)
    lens = np.array(wl.lengths_q)
    order = np.argsort(lens)
    seqs = [int(order[0]), int(order[len(order) // 3]), int(order[len(order) // 2]),
            int(order[(2 * len(order)) // 3])]
    heads = [0, 17]
    ref = attention_bwd(data["q"], data["k"], data["v"], g["dout"], wl.cu_q, wl.cu_k, wl.scale, True,
                        heads=heads, seqs=seqs)
    # dq: compared on the chosen heads; dk/dv: kv head == query head here (no sharing)
    sel = [got[0][:, heads], got[1][:, heads], got[2][:, heads]]
    refs = [ref[0][:, heads], ref[1][:, heads], ref[2][:, heads]]
    compare_grads(sel, refs, wl.dtype, wl.name)
    for x in got:
        assert not np.isnan(x[:wl.total_q]).any()


def test_bwd_dk_dv_deterministic_and_workspace_contents_ignored(fa):
    wl = workload_custom("bwd_det_h4_d128", [300, 129, 700], None, 4, 128, "bf16", seed=24)
    need = fa.fa_varlen_bwd_workspace_size(wl.batch, wl.total_q, wl.heads, wl.head_dim)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN patterns everywhere
    _, _, a = run_fwd_bwd(fa, wl, True, workspace=ws)
    _, _, b = run_fwd_bwd(fa, wl, True)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]), "dk/dv must not depend on the run"
    assert not np.isnan(a[0]).any()
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-2)
