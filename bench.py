#!/usr/bin/env python3
"""Benchmark of exact varlen attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch: the work-item map and
the attention kernel, i.e. one fa_varlen_fwd call through the C ABI, with
Q/K/V, the offsets and the outputs already resident in HBM.  The headline
workload is the heavily ragged causal batch (65,536 tokens in sequences of
log-uniform length 64..8192, 32 heads of dimension 128, bf16, seed 4).

Prints ONE JSON line with: the throughput in TFLOP/s of algorithmic work
(4 * head_dim flops per visible (query, key) pair per head -- two for the
score, two for the probability-weighted value; masked pairs and the softmax
are not counted); the attention kernel's own roofline fraction, timed with
HIP events on the stream it is launched on; the oracle's rate on the host
cores on a bounded sample (``cpu_baseline``); and secondary rows for the
16k-token sequence-length sweep (head dim 64 and 128, causal and not) and
the dense 8x2048 batch.

Counter mode (``--pmc-pass``) runs a short fixed sequence for rocprofv3 --pmc:
a plain device copy of known size (to calibrate FETCH_SIZE / WRITE_SIZE)
followed by attention launches; ``--parse-pmc DIR`` turns the two counter
runs into per-launch HBM bytes stored under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
import hashlib
import json
import math
import sqlite3
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fa_synth import (SWEEP_HEAD_DIMS, SWEEP_SEQLENS, Workload, draw_dout, draw_qkv, workload_dense,  # noqa: E402
                      workload_ragged64k, workload_ragged64k_gqa, workload_sweep, draw_kvcache,
                      workload_decode_bench)

METRIC = "varlen attention fwd TFLOP/s and % of bf16 MFMA peak, d=64/128, causal"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
CSRC_DIR = os.path.join(ROOT, "variable_length_flashattention_cu_amd", "csrc")
# the forward kernels' source and every header it includes
KERNEL_SRCS = [os.path.join(CSRC_DIR, n) for n in
               ("fa_varlen_kernels.hip", "fa_varlen_device.h", "fa_varlen_tiling.h", "fa_varlen_launch.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_ragged64k_causal_d128.json")
COPY_BYTES = 1 << 30        # calibration copy: 1 GiB read + 1 GiB written
FWD_KERNEL_TAG = "fwd16_"   # name fragment of the 16-bit forward attention kernels


def visible_pairs(wl: Workload, causal: bool) -> int:
    """Visible (query, key) pairs per head; bottom-right causal alignment."""
    total = 0
    for Lq, Lk in zip(wl.lengths_q, wl.lengths_k):
        if not causal:
            total += Lq * Lk
            continue
        # row i sees clip(i + Lk - Lq + 1, 0, Lk) keys
        s = Lk - Lq + 1
        i = np.arange(Lq, dtype=np.int64)
        total += int(np.clip(i + s, 0, Lk).sum())
    return total


def algorithmic_flops(wl: Workload, causal: bool) -> float:
    return 4.0 * wl.head_dim * wl.heads * visible_pairs(wl, causal)


def algorithmic_bytes(wl: Workload) -> float:
    """Q, K, V read once and out, lse written once (K/V with the key/value head count)."""
    es = 4 if wl.dtype == "f32" else 2
    hd, hkd = wl.heads * wl.head_dim, wl.kv_heads * wl.head_dim
    return float(2 * wl.total_q * hd * es + 2 * wl.total_k * hkd * es + 4 * wl.total_q * wl.heads)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def to_device(wl: Workload, data: dict):
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    t = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).to("cuda").view(tdt) for n in "qkv"}
    t["cu_q"] = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    t["cu_k"] = torch.tensor(wl.cu_k, dtype=torch.int32, device="cuda")
    H, Tq = wl.heads, wl.total_q
    t["out"] = torch.empty_like(t["q"])
    t["lse"] = torch.empty((H, Tq), dtype=torch.float32, device="cuda")
    return t


class Runner:
    """Calls the C ABI with preallocated buffers and descriptors on torch's current stream."""

    def __init__(self, wl: Workload, t: dict, causal: bool):
        import ctypes
        import torch
        import variable_length_flashattention_cu_amd as fa
        self.fa, self.wl, self.t, self.causal = fa, wl, t, causal
        self.lib = fa.load_library()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.dt = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[wl.dtype]
        self.blk = fa.fa_varlen_tile_map(t["cu_q"], wl.max_seqlen_q, wl.head_dim, self.dt)
        self.descs = [fa.desc(t[n]) for n in ("q", "k", "v", "cu_q", "cu_k", "out", "lse")] + [fa.desc(self.blk)]
        r = [ctypes.byref(d) for d in self.descs]
        self.args = (r[0], r[1], r[2], r[3], r[4], wl.max_seqlen_q, wl.max_seqlen_k, ctypes.c_float(wl.scale),
                     int(causal), r[5], r[6])
        self.blk_ref = r[7]

    def step(self):
        st = self.lib.fa_varlen_fwd(*self.args, self.stream)
        if st:
            raise RuntimeError(f"fa_varlen_fwd failed: {self.fa.fa_status_string(st)}")

    def kernel_only(self):
        st = self.lib.fa_varlen_fwd_mapped(*self.args, self.blk_ref, self.stream)
        if st:
            raise RuntimeError(f"fa_varlen_fwd_mapped failed: {self.fa.fa_status_string(st)}")


# ---------------------------------------------------------------------------
# timing: a time-based pre-warm, then HIP events on torch's current stream
# (the stream every call here is launched on)
# ---------------------------------------------------------------------------
PREWARM_MS = 200.0   # wall time of untimed calls before every timed loop
MIN_TIMED_MS = 200.0
MIN_TIMED_CALLS = 50


def prewarm(fn, min_ms: float = PREWARM_MS) -> dict:
    """Call fn until at least min_ms of wall time has passed (synchronised)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0 or n < 4:
            torch.cuda.synchronize()
            el = (time.perf_counter() - t0) * 1e3
            if el >= min_ms:
                return {"calls": n, "ms": round(el, 1)}


def per_call_ms(fn, iters: int) -> np.ndarray:
    """Per-call milliseconds: one event pair around every call."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev], dtype=np.float64)


def bracketed_ms(fn, iters: int) -> float:
    """Mean milliseconds per call of `iters` back-to-back calls between two events."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def timed_iters(pw: dict) -> int:
    """At least MIN_TIMED_CALLS calls and MIN_TIMED_MS of device time, from the pre-warm rate."""
    per = pw["ms"] / max(pw["calls"], 1)
    return int(max(MIN_TIMED_CALLS, math.ceil(MIN_TIMED_MS / max(per, 1e-3))))


def call_stats(ms: np.ndarray) -> dict:
    return {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(ms.min()), 4),
            "mean_ms": round(float(ms.mean()), 4), "calls": int(ms.size)}


# ---------------------------------------------------------------------------
# sampled outputs for the parity check (rows chosen without the oracle)
# ---------------------------------------------------------------------------
def sample_rows(wl: Workload, block: int = 256, per_seq: int = 4, seed: int = 0) -> np.ndarray:
    """Packed query rows: the first and last row of every sequence and of every
    block of `block` rows (one query block of the forward kernel), plus a few
    random rows per sequence."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(wl.batch):
        s, L = wl.cu_q[b], wl.cu_q[b + 1] - wl.cu_q[b]
        if L <= 0:
            continue
        cand = {0, L - 1} | {int(x) for x in rng.integers(0, L, size=per_seq)}
        for m0 in range(0, L, block):
            cand |= {m0, min(L - 1, m0 + block - 1)}
        rows |= {s + c for c in cand}
    return np.array(sorted(rows), dtype=np.int64)


def take_sample(wl: Workload, t: dict, causal: bool, heads) -> dict:
    import torch
    rows = sample_rows(wl, seed=wl.seed)
    idx = torch.from_numpy(rows).to(t["out"].device)
    hs = torch.tensor(list(heads), device=t["out"].device)
    out = t["out"].index_select(0, idx).index_select(1, hs).float().cpu().numpy()
    lse = t["lse"].index_select(0, hs).index_select(1, idx).cpu().numpy()
    return {"rows": rows, "heads": list(heads), "out": out, "lse": lse, "causal": causal}


def call_block_m(wl: Workload) -> int:
    """Query rows per work item of a whole fa_varlen_fwd call: 128 for 16-bit
    inputs at head_dim 64/128 with max_seqlen_q <= 1024 (the library's short
    configuration), else the BM of fa_varlen_block_sizes, which the mapped
    (kernel-only) entry point always uses."""
    import variable_length_flashattention_cu_amd as fa
    if wl.dtype in ("bf16", "f16") and wl.head_dim in (64, 128) and wl.max_seqlen_q <= 1024:
        return 128
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[wl.dtype]
    return fa.fa_varlen_block_sizes(wl.head_dim, code)[0]


def measure_fwd(wl: Workload, t: dict, causal: bool) -> tuple:
    """One forward workload: whole-call and kernel-only per-call times, and a
    sample of the outputs for the parity check.  The kernel-only figure times
    fa_varlen_fwd_mapped (work items of fa_varlen_block_sizes' BM); for short
    batches the whole call runs 128-row items instead (`call_block_m`)."""
    r = Runner(wl, t, causal)
    pw = prewarm(r.step)
    n = timed_iters(pw)
    call = call_stats(per_call_ms(r.step, n))
    pwk = prewarm(r.kernel_only)
    kern = call_stats(per_call_ms(r.kernel_only, n))
    fl = algorithmic_flops(wl, causal)
    by = algorithmic_bytes(wl)
    row = {"workload": wl.name, "seq_len": wl.max_seqlen_q, "head_dim": wl.head_dim, "heads": wl.heads,
           "kv_heads": wl.kv_heads, "dtype": wl.dtype, "causal": causal, "seed": wl.seed,
           "gflop": round(fl / 1e9, 3), "algorithmic_mb": round(by / 1e6, 2),
           "prewarm": pw, "call": call, "kernel": kern,
           "tflops": round(fl / call["median_ms"] / 1e9, 1),
           "kernel_tflops": round(fl / kern["median_ms"] / 1e9, 1),
           "kernel_frac_bf16_peak": round(fl / kern["median_ms"] / 1e9 / PEAK_BF16_TFLOPS, 4),
           "kernel_frac_hbm_peak": round(by / kern["median_ms"] / 1e6 / PEAK_HBM_GBS, 4),
           "kernel_prewarm": pwk,
           "call_frac_bf16_peak": round(fl / call["median_ms"] / 1e9 / PEAK_BF16_TFLOPS, 4),
           "call_block_m": call_block_m(wl)}
    sample = take_sample(wl, t, causal, sorted({0, wl.heads - 1}))
    del r
    return row, sample


def measure_secondary(wl: Workload, modes=(False, True), parity=None) -> list:
    """The given mask modes of one workload (inputs drawn once)."""
    data = draw_qkv(wl)
    t = to_device(wl, data)
    rows = []
    for causal in modes:
        row, sample = measure_fwd(wl, t, causal)
        if parity is not None:
            row["parity"] = parity(wl, data, sample)
        rows.append(row)
    del t, data
    return rows


def measure_backward(wl: Workload, causal: bool) -> dict:
    """fa_varlen_bwd (all four launches) after one forward; 10*D flops per
    visible pair and head (S recomputed, dP, dV, dK, dQ: five products)."""
    import torch
    import variable_length_flashattention_cu_amd as fa
    data = draw_qkv(wl)
    t = to_device(wl, data)
    del data
    g = draw_dout(wl)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    dout = torch.from_numpy(g["dout_bits"].view(np.int16)).to("cuda").view(tdt)
    del g
    out, lse = fa.fa_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                wl.scale, causal)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ws = torch.empty(fa.fa_varlen_bwd_workspace_size(wl.batch, wl.total_q, wl.heads, wl.head_dim),
                     dtype=torch.uint8, device="cuda")

    def step():
        fa.fa_varlen_bwd(t["q"], t["k"], t["v"], out, dout, lse, t["cu_q"], t["cu_k"], wl.max_seqlen_q,
                         wl.max_seqlen_k, wl.scale, causal, dq=dq, dk=dk, dv=dv, workspace=ws)
    pw = prewarm(step)
    call = call_stats(per_call_ms(step, timed_iters(pw)))
    fl = 2.5 * algorithmic_flops(wl, causal)
    return {"workload": wl.name, "seq_len": wl.max_seqlen_q, "head_dim": wl.head_dim, "heads": wl.heads,
            "kv_heads": wl.kv_heads, "dtype": wl.dtype, "causal": causal, "prewarm": pw, "call": call,
            "tflops": round(fl / call["median_ms"] / 1e9, 1),
            "frac_bf16_peak": round(fl / call["median_ms"] / 1e9 / PEAK_BF16_TFLOPS, 4)}


def measure_decode(wl) -> dict:
    """fa_varlen_fwd_kvcache (decode kernel and partial combine) on a cache batch.
    Algorithmic bytes: the cached K and V rows each sequence uses (once per
    key/value head), q read, out and lse written."""
    import torch
    import variable_length_flashattention_cu_amd as fa
    data = draw_kvcache(wl)
    tt = {"bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    dev = {n: torch.from_numpy(data[n + "_bits"].view(np.int16)).to("cuda").view(tt)
           for n in ("q", "k_cache", "v_cache")}
    bt = torch.from_numpy(data["block_table"]).to("cuda") if wl.paged else None
    del data
    cu_q = torch.tensor(wl.cu_q, dtype=torch.int32, device="cuda")
    sk = torch.tensor(wl.seqlens_k, dtype=torch.int32, device="cuda")
    lp = None if wl.leftpad is None else torch.tensor(wl.leftpad, dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((wl.heads, wl.total_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_varlen_kvcache_workspace_size(wl.total_q, wl.heads, wl.head_dim, 0), dtype=torch.uint8,
                     device="cuda")

    def step():
        fa.fa_varlen_fwd_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], cu_q, sk, wl.max_seqlen_q,
                                 wl.max_seqlen_k, wl.scale, True, leftpad_k=lp, block_table=bt, out=out, lse=lse,
                                 workspace=ws)
    pw = prewarm(step)
    call = call_stats(per_call_ms(step, timed_iters(pw)))
    ms = call["median_ms"]
    es = 2
    kv_bytes = 2.0 * sum(wl.key_lengths) * wl.kv_heads * wl.head_dim * es
    qo_bytes = 2.0 * wl.total_q * wl.heads * wl.head_dim * es + 4.0 * wl.total_q * wl.heads
    gbs = (kv_bytes + qo_bytes) / ms / 1e6
    return {"workload": wl.name, "batch": wl.batch, "kv_tokens": int(sum(wl.key_lengths)), "heads": wl.heads,
            "kv_heads": wl.kv_heads, "head_dim": wl.head_dim, "dtype": wl.dtype, "prewarm": pw, "call": call,
            "algorithmic_bytes": round(kv_bytes + qo_bytes), "gb_per_s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


# ---------------------------------------------------------------------------
# cpu_baseline leg: the oracle on the host cores -- its timed sample, and the
# sampled parity checks of the measured GPU outputs (only this leg runs it)
# ---------------------------------------------------------------------------
def cpu_parity(wl: Workload, data: dict, sample: dict) -> dict:
    """Max-abs difference of the sampled GPU rows and heads against the oracle."""
    from oracle import attention_rows
    tol = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}[wl.dtype]
    ref_o, ref_l = attention_rows(data["q"], data["k"], data["v"], wl.cu_q, wl.cu_k, wl.scale, sample["causal"],
                                  sample["rows"], sample["heads"])
    fin = np.isfinite(ref_l)
    err_o = float(np.abs(sample["out"].astype(np.float64) - ref_o).max()) if ref_o.size else 0.0
    err_l = float(np.abs(sample["lse"][fin].astype(np.float64) - ref_l[fin]).max()) if fin.any() else 0.0
    pattern = bool(np.array_equal(np.isfinite(sample["lse"]), fin))
    ok = err_o <= tol and err_l <= tol and pattern and not np.isnan(sample["out"]).any()
    return {"rows": int(sample["rows"].size), "heads": sample["heads"], "max_abs_out": float(f"{err_o:.3e}"),
            "max_abs_lse": float(f"{err_l:.3e}"), "tol": tol, "ok": bool(ok)}


def cpu_baseline(wl: Workload, causal: bool, data: dict, min_seconds: float = 10.0) -> dict:
    """The oracle (float64 numpy) on a bounded sample: whole heads (every
    sequence), one at a time, until about `min_seconds` of CPU work."""
    from threadpoolctl import threadpool_info
    from oracle import attention_fwd
    group = wl.heads // (wl.heads_k or wl.heads)
    heads, dt = [], 0.0
    for h in range(wl.heads):
        sub = {"q": np.ascontiguousarray(data["q"][:, [h], :])}
        for n in "kv":
            sub[n] = np.ascontiguousarray(data[n][:, [h // group], :])
        t0 = time.perf_counter()
        attention_fwd(sub["q"], sub["k"], sub["v"], wl.cu_q, wl.cu_k, wl.scale, causal)
        dt += time.perf_counter() - t0
        heads.append(h)
        if dt >= min_seconds:
            break
    fl = 4.0 * wl.head_dim * len(heads) * visible_pairs(wl, causal)
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "blas_threads": int(threads),
            "blas": (blas[0].get("internal_api", "?") if blas else "?"),
            "sample": f"{wl.name}: heads {heads[0]}-{heads[-1]} of {wl.heads}, all {wl.batch} sequences "
                      f"({fl / 1e9:.1f} GFLOP algorithmic, {dt:.1f} s, float64 numpy on {threads} BLAS threads "
                      f"of {os.cpu_count()} host cores)"}


def stored_traffic() -> dict | None:
    """Per-launch HBM bytes from the committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec


# ---------------------------------------------------------------------------
# counter runs
# ---------------------------------------------------------------------------
def pmc_pass(steps: int) -> None:
    """Fixed launch sequence for rocprofv3 --pmc: one calibration copy, then attention."""
    import torch
    wl = workload_ragged64k()
    data = draw_qkv(wl)
    t = to_device(wl, data)
    del data
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # elementwise copy kernel: COPY_BYTES read, COPY_BYTES written
    torch.cuda.synchronize()
    del src, dst
    r = Runner(wl, t, True)
    for _ in range(steps):
        r.kernel_only()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": "done", "launches": steps}), flush=True)


def _counter_per_dispatch(run_dir: str, counter: str) -> dict:
    """{(kernel_name, dispatch_id): value} from a rocprofv3 run (rocpd database or CSV)."""
    out: dict = {}
    dbs = glob.glob(os.path.join(run_dir, "**", "*results.db"), recursive=True)
    for db in dbs:
        con = sqlite3.connect(db)
        q = ("select kernel_name, dispatch_id, sum(value) from counters_collection "
             "where counter_name = ? group by kernel_name, dispatch_id")
        for name, disp, val in con.execute(q, (counter,)):
            out[(name, (db, disp))] = float(val)
        con.close()
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    key = (row["Kernel_Name"], (path, row["Dispatch_Id"]))
                    out[key] = out.get(key, 0.0) + float(row["Counter_Value"])
    return out


def parse_pmc(fetch_dir: str, write_dir: str) -> dict:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> calibrated bytes per attention launch.

    Each counter is scaled by COPY_BYTES divided by what the same counter reads
    for the calibration copy (an elementwise kernel reading and writing
    COPY_BYTES), in the same process."""
    out = {"kernel_sha": kernel_sha(), "workload": workload_ragged64k().name, "copy_bytes": COPY_BYTES,
           "command": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE -- python bench.py --pmc-pass --steps 3"}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per_disp = _counter_per_dispatch(d, counter)
        copy_vals = [v for (k, _), v in per_disp.items() if "elementwise" in k.lower()]
        fwd_vals = [v for (k, _), v in per_disp.items() if FWD_KERNEL_TAG in k]
        if not copy_vals or not fwd_vals:
            raise RuntimeError(f"{counter}: calibration copy or attention dispatches not found in {d}")
        copy_kib = max(copy_vals)
        factor = (COPY_BYTES / 1024.0) / copy_kib
        fwd_kib = float(np.mean(fwd_vals))
        out[counter] = {"raw_kib_per_launch": round(fwd_kib, 1), "copy_raw_kib": round(copy_kib, 1),
                        "scale_factor": round(factor, 4), "bytes_per_launch": round(fwd_kib * 1024.0 * factor),
                        "launches": len(fwd_vals)}
    out["traffic_bytes"] = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    out["algorithmic_bytes"] = round(algorithmic_bytes(workload_ragged64k()))
    return out


def summarize_trace(db_path: str, last: int = 100) -> str:
    """Per-kernel call count / total / average duration from a --kernel-trace run."""
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    con.close()
    # the top_kernels view reports microseconds
    lines = [f"{'calls':>6} {'total_ms':>10} {'avg_us':>10} {'pct':>6}  kernel"]
    for name, calls, tot, avg, pct in rows:
        lines.append(f"{calls:>6} {tot / 1e3:>10.3f} {avg:>10.2f} {pct:>6.2f}  {name}")
    # per-dispatch durations of the attention kernel: the first launches of a
    # process are cold (code and data not yet cached), so the median and the
    # mean without the first two are what compares with the timed steps
    con = sqlite3.connect(db_path)
    durs = [r[0] for r in con.execute(f"select duration from kernels where name like '%{FWD_KERNEL_TAG}%' "
                                      "order by start")]
    con.close()
    if durs:
        us = np.asarray(durs, dtype=np.float64) / 1e3  # nanoseconds -> microseconds
        warm = us[10:] if len(us) > 10 else us
        lines.append(f"attention kernel, {len(us)} dispatches: first {us[0]:.1f} us; after the first ten: "
                     f"median {np.median(warm):.1f} us, mean {warm.mean():.1f} us")
        if len(us) >= last:
            tail = us[-last:]
            lines.append(f"the last {last} dispatches (the timed kernel-only loop of the bench run): "
                         f"mean {tail.mean():.1f} us, median {np.median(tail):.1f} us, min {tail.min():.1f} us")
    return "\n".join(lines)


# ---------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the sweep and dense rows")
    ap.add_argument("--pmc-pass", action="store_true", help="launch sequence for a rocprofv3 --pmc run")
    ap.add_argument("--decode-pass", action="store_true",
                    help="only the key/value-cache decode batch (for profiling)")
    ap.add_argument("--bwd-pass", action="store_true",
                    help="only the backward pass of the 64k ragged causal batch (for profiling)")
    ap.add_argument("--parse-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB", help="print kernel stats of a rocprofv3 trace")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the forward pass runs on one GPU and is not sharded across GPUs", file=sys.stderr)
        return 2
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.parse_pmc:
        rec = parse_pmc(*args.parse_pmc)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.decode_pass:
        print(json.dumps(measure_decode(workload_decode_bench())), flush=True)
        return 0
    if args.bwd_pass:
        print(json.dumps(measure_backward(workload_ragged64k(), True)), flush=True)
        return 0
    if args.pmc_pass:
        pmc_pass(max(1, args.steps))
        return 0

    import torch
    wl = workload_ragged64k()
    causal = True
    print(f"# bench: {wl.name} batch={wl.batch} tokens={wl.total_q} heads={wl.heads} d={wl.head_dim} "
          f"causal={causal}", file=sys.stderr, flush=True)
    props = torch.cuda.get_device_properties(0)
    gpu = {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", "?"),
           "compute_units": props.multi_processor_count, "memory_gb": round(props.total_memory / 2**30, 1)}
    ceiling = mfma_ceiling()
    print(f"# gpu {gpu}; measured MFMA ceiling {ceiling}", file=sys.stderr, flush=True)

    data = draw_qkv(wl)
    t = to_device(wl, data)
    torch.cuda.reset_peak_memory_stats()
    r = Runner(wl, t, causal)
    for _ in range(args.warmup):
        r.step()
    pw = prewarm(r.step)
    # the headline: exactly `steps` whole calls between two synchronisations
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ms = bracketed_ms(r.step, args.steps)
    wall = (time.perf_counter() - w0) * 1e3 / args.steps
    call = call_stats(per_call_ms(r.step, args.steps))
    pwk = prewarm(r.kernel_only)
    kern = call_stats(per_call_ms(r.kernel_only, args.steps))
    peak_mem = torch.cuda.max_memory_allocated()
    fl = algorithmic_flops(wl, causal)
    value = fl / ms / 1e9
    achieved = fl / kern["mean_ms"] / 1e9
    print(f"# step {ms:.3f} ms ({value:.1f} TFLOP/s), attention kernel mean {kern['mean_ms']:.4f} ms "
          f"median {kern['median_ms']:.4f} ms ({achieved:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    sample = take_sample(wl, t, causal, [0, wl.heads // 2, wl.heads - 1])

    traffic = stored_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "total_tokens": wl.total_q, "batch": wl.batch,
                   "seq_len_range": [min(wl.lengths_q), max(wl.lengths_q)], "heads": wl.heads,
                   "head_dim": wl.head_dim, "causal": causal, "seed": wl.seed,
                   "gflop_per_step": round(fl / 1e9, 2), "wall_ms_per_step": round(wall, 4)},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": round(traffic["traffic_bytes"]) if traffic else None,
                     "kernel": "fwd16 attention kernel <__bf16, 128, causal>", "kernel_ms": kern["mean_ms"],
                     "kernel_ms_median": kern["median_ms"], "kernel_ms_min": kern["min_ms"],
                     "algorithmic_bytes": round(algorithmic_bytes(wl)),
                     "frac_of_measured_mfma_ceiling": (round(achieved / ceiling["tflops"], 4)
                                                       if ceiling.get("tflops") else None),
                     "frac_of_random_operand_mfma_ceiling": (
                         round(achieved / ceiling["random_operands"]["tflops"], 4)
                         if ceiling.get("random_operands", {}).get("tflops") else None)},
        "timing": {"prewarm_call": pw, "prewarm_kernel": pwk, "call": call, "kernel": kern,
                   "method": "HIP events on the launch stream after a >=200 ms pre-warm; value from `steps` "
                             "back-to-back calls between two synchronisations"},
        "gpu": gpu,
        "mfma_ceiling": ceiling,
        "peak_memory_bytes": int(peak_mem),
    }
    del r
    t = None
    torch.cuda.empty_cache()
    par = None if args.no_cpu_baseline else cpu_parity

    if not args.no_secondary:
        rows = []
        for d in SWEEP_HEAD_DIMS:
            for L in SWEEP_SEQLENS:
                rows += measure_secondary(workload_sweep(L, d), parity=par)
                for row in rows[-2:]:
                    print(f"# {row}", file=sys.stderr, flush=True)
                torch.cuda.empty_cache()
        line["sweep_16k_tokens"] = rows
        line["dense_8x2048"] = measure_secondary(workload_dense(), parity=par)
        torch.cuda.empty_cache()
        # the headline length mix with fp16 inputs, 8 shared key/value heads, head_dim 96 and 256
        base = workload_ragged64k()
        variants = [dataclasses.replace(base, name=base.name.replace("_h32_", "_h32_f16_"), dtype="f16"),
                    workload_ragged64k_gqa(),
                    dataclasses.replace(base, name=base.name.replace("_d128_", "_d96_"), head_dim=96),
                    dataclasses.replace(base, name=base.name.replace("_h32_d128_", "_h16_d256_"), heads=16,
                                        head_dim=256)]
        line["ragged64k_variants"] = []
        for v in variants:
            line["ragged64k_variants"] += measure_secondary(v, modes=(True,), parity=par)
            print(f"# {line['ragged64k_variants'][-1]}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        # backward pass (fa_varlen_bwd, after the forward that gives out and lse)
        line["backward"] = []
        base = workload_ragged64k()
        for bwl, bc in ((base, True), (workload_sweep(4096, 128), False),
                        (workload_sweep(4096, 128), True), (workload_sweep(4096, 64), True),
                        (dataclasses.replace(base, name=base.name.replace("_d128_", "_d96_"), head_dim=96), True),
                        (dataclasses.replace(base, name=base.name.replace("_h32_d128_", "_h16_d256_"), heads=16,
                                             head_dim=256), True)):
            line["backward"].append(measure_backward(bwl, bc))
            print(f"# {line['backward'][-1]}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        # decode-shaped attention against a paged key/value cache (HBM-bound)
        line["decode"] = measure_decode(workload_decode_bench())
        print(f"# {line['decode']}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        line["parity"] = cpu_parity(wl, data, sample)
        line["cpu_baseline"] = cpu_baseline(wl, causal, data)
    print(json.dumps(line), flush=True)
    return 0


def mfma_ceiling() -> dict:
    """Dense bf16 MFMA rate of a register-only loop on this device (libfa_probe.so)."""
    import ctypes
    path = os.path.join(ROOT, "variable_length_flashattention_cu_amd", "libfa_probe.so")
    if not os.path.exists(path):
        return {"tflops": None, "note": "libfa_probe.so not built"}
    lib = ctypes.CDLL(path)
    lib.fa_probe_mfma_peak.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
    lib.fa_probe_mfma_peak.restype = ctypes.c_int
    lib.fa_probe_mfma_peak_random.argtypes = [ctypes.c_int32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_double)]
    lib.fa_probe_mfma_peak_random.restype = ctypes.c_int
    tf, ghz = ctypes.c_double(0), ctypes.c_double(0)
    best = {}
    for name, call in (("constant", lambda: lib.fa_probe_mfma_peak(20000, ctypes.byref(tf), ctypes.byref(ghz))),
                       ("random", lambda: lib.fa_probe_mfma_peak_random(20000, 12345, ctypes.byref(tf),
                                                                         ctypes.byref(ghz)))):
        for _ in range(3):
            rc = call()
            if rc != 0:
                return {"tflops": None, "note": f"probe failed with status {rc}"}
            if name not in best or tf.value > best[name][0]:
                best[name] = (tf.value, ghz.value)
    c, r = best["constant"], best["random"]
    return {"tflops": round(c[0], 1), "clock_ghz": round(c[1], 3),
            "frac_of_published_peak": round(c[0] / PEAK_BF16_TFLOPS, 4),
            "method": "v_mfma_f32_32x32x16_bf16 on registers, 2 waves per SIMD on every CU, best of 3",
            "random_operands": {"tflops": round(r[0], 1), "clock_ghz": round(r[1], 3),
                                "frac_of_published_peak": round(r[0] / PEAK_BF16_TFLOPS, 4),
                                "method": "the same loop on pseudo-random bf16 operands, 8 operand pairs per wave"}}


if __name__ == "__main__":
    sys.exit(main())
