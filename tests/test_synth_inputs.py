"""Seeded input generation: bf16 rounding and workload shapes (CPU)."""
import numpy as np
import torch

from fa_synth import (SWEEP_HEAD_DIMS, SWEEP_SEQLENS, all_parity_workloads, bf16_bits_to_f32,
                      bf16_rne_bits, cu_from_lengths, draw_qkv, f16_bits_to_f32, f16_rne_bits,
                      workload_custom, workload_ragged64k, workload_ragged64k_gqa, workload_ragged_qk,
                      workload_sweep, workload_tiny)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-3, 3),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e38], dtype=np.float32)])
    x = x.astype(np.float32)
    ours = bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert bf16_bits_to_f32(bf16_rne_bits(np.array([1.00390625], np.float32)))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: goes to 1 + 2^-6 (even)
    assert bf16_bits_to_f32(bf16_rne_bits(np.array([1.01171875], np.float32)))[0] == 1.015625


def test_workload_shapes():
    t = workload_tiny()
    assert t.cu_q == (0, 128, 300) and t.heads == 2 and t.head_dim == 64 and t.dtype == "f32"
    r = workload_ragged_qk()
    assert r.lengths_q == [200, 824] and r.lengths_k == [300, 724] and r.heads == 12
    for L in SWEEP_SEQLENS:
        for d in SWEEP_HEAD_DIMS:
            w = workload_sweep(L, d)
            assert w.total_q == 16384 and w.heads * d == 2048 and w.batch * L == 16384
    g = workload_ragged64k()
    lens = g.lengths_q
    assert sum(lens) == 65536 and all(64 <= L <= 8192 for L in lens[:-1]) and 1 <= lens[-1] <= 8192
    assert g.heads == 32 and g.head_dim == 128 and g.causal_modes == (True,)
    assert len({w.name for w in all_parity_workloads()}) == len(all_parity_workloads())


def test_draws_are_seeded_and_bf16_exact():
    w = workload_ragged_qk()
    a = draw_qkv(w)
    b = draw_qkv(w)
    for n in "qkv":
        assert np.array_equal(a[n], b[n])
        assert np.array_equal(bf16_bits_to_f32(a[n + "_bits"]).reshape(a[n].shape), a[n])
    sub = draw_qkv(w, heads=[0, 11])
    assert np.array_equal(sub["q"], a["q"][:, [0, 11]]) and np.array_equal(sub["k"], a["k"])
    assert abs(float(a["q"].mean())) < 0.01 and abs(float(a["q"].std()) - 1) < 0.01


def test_cu_from_lengths():
    assert cu_from_lengths([128, 172]).tolist() == [0, 128, 300]
    assert cu_from_lengths([]).tolist() == [0]


def test_f16_rounding_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-4, 4, 100000)).astype(np.float32)
    x = np.concatenate([x, np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 70000.0, 1e-6], np.float32)])
    ours = f16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # 1 + 2^-11 is halfway between fp16 1.0 and 1 + 2^-10: ties to even (1.0)
    assert f16_bits_to_f32(f16_rne_bits(np.array([1.0 + 2 ** -11], np.float32)))[0] == 1.0
    assert f16_bits_to_f32(f16_rne_bits(np.array([1.0 + 3 * 2 ** -11], np.float32)))[0] == 1.0 + 2 ** -9


def test_gqa_and_f16_workloads():
    w = workload_custom("g", [100, 37], [90, 50], 8, 64, "f16", 3, heads_k=2)
    d = draw_qkv(w)
    assert d["q"].shape == (137, 8, 64) and d["k"].shape == (140, 2, 64) and d["v"].shape == (140, 2, 64)
    for n in "qkv":
        assert d[n + "_bits"].dtype == np.uint16
        assert np.array_equal(f16_bits_to_f32(d[n + "_bits"]).reshape(d[n].shape), d[n])
    g = workload_ragged64k_gqa()
    assert g.kv_heads == 8 and g.heads == 32 and g.cu_q == workload_ragged64k().cu_q
    import pytest
    with pytest.raises(ValueError):
        workload_custom("bad", [4], None, 6, 64, "bf16", 0, heads_k=4)


def test_dout_is_seeded_rounded_and_separate_from_qkv():
    from fa_synth import bf16_bits_to_f32, draw_dout
    wl = workload_ragged_qk()
    a, b = draw_dout(wl), draw_dout(wl)
    assert np.array_equal(a["dout_bits"], b["dout_bits"])
    assert np.array_equal(bf16_bits_to_f32(a["dout_bits"]).reshape(a["dout"].shape), a["dout"])
    qkv = draw_qkv(wl)
    assert a["dout"].shape == qkv["q"].shape and not np.array_equal(a["dout"], qkv["q"])
    assert abs(float(a["dout"].std()) - 1.0) < 0.02
