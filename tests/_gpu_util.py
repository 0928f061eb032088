"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, and compare with the oracle."""
import sys

import numpy as np

# max-abs bounds: bf16 and fp32 from the stated parity bar; fp16 derived from
# its rounding (output rounded to fp16: <= 2^-9 for |out| < 4; probabilities
# rounded to fp16 before the second product: <= 2^-11 relative per weight,
# <= 2e-3 on an average of values below 4), with margin.
TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}


def dtype_code(fa, name):
    """fa_dtype code of a workload dtype name."""
    return {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[name]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(data, wl):
    import torch
    dev = "cuda"
    if wl.dtype in ("bf16", "f16"):
        tt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        t = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).to(dev).view(tt) for n in "qkv"}
    else:
        t = {n: torch.from_numpy(data[n]).to(dev) for n in "qkv"}
    t["cu_q"] = torch.tensor(wl.cu_q, dtype=torch.int32, device=dev)
    t["cu_k"] = torch.tensor(wl.cu_k, dtype=torch.int32, device=dev)
    return t


def run_gpu(wl, t, causal, out=None, lse=None):
    import torch
    import variable_length_flashattention_cu_amd as fa
    o, l = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                            wl.scale, causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


def host(o, l):
    return o.float().cpu().numpy(), l.cpu().numpy()


def sample_rows(wl, bm, rng, per_seq=6):
    """Packed query rows that exercise sequence starts/ends, tile edges and random interiors."""
    rows = set()
    for b in range(wl.batch):
        s, L = wl.cu_q[b], wl.cu_q[b + 1] - wl.cu_q[b]
        if L == 0:
            continue
        cand = {0, L - 1, min(L - 1, bm - 1), min(L - 1, bm), L // 2}
        cand |= {int(x) for x in rng.integers(0, L, size=per_seq)}
        rows |= {s + c for c in cand}
    return np.array(sorted(rows), dtype=np.int64)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, tol, what=""):
    """Max-abs comparison of out (valid rows) and finite lse; -inf must match exactly."""
    assert out_gpu.shape == out_ref.shape and lse_gpu.shape == lse_ref.shape, what
    assert not np.isnan(out_gpu).any(), f"{what}: NaN in out"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in lse"
    err_o = float(np.max(np.abs(out_gpu.astype(np.float64) - out_ref))) if out_ref.size else 0.0
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: finite-lse pattern differs"
    assert np.all(lse_gpu[~fin] == -np.inf), f"{what}: rows with no visible key must have lse=-inf"
    err_l = float(np.max(np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin]))) if fin.any() else 0.0
    say(f"  {what}: max|dout|={err_o:.3e} max|dlse|={err_l:.3e} (tol {tol:g})")
    assert err_o <= tol, f"{what}: out error {err_o} > {tol}"
    assert err_l <= tol, f"{what}: lse error {err_l} > {tol}"
    return err_o, err_l
