"""The bench's FLOP and byte accounting (CPU): its closed-form visible-pair
count must equal the count taken from the oracle's mask."""
import numpy as np
import pytest

import bench
from fa_synth import workload_custom, workload_dense, workload_ragged64k, workload_ragged_qk, workload_sweep
from oracle import flops_visible_pairs


@pytest.mark.parametrize("wl", [workload_ragged_qk(), workload_dense(), workload_sweep(512, 64),
                                workload_custom("odd", [5, 0, 300, 1], [7, 3, 250, 40], 1, 64, "bf16", 0)],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_match_oracle_mask(wl, causal):
    assert bench.visible_pairs(wl, causal) == flops_visible_pairs(wl.cu_q, wl.cu_k, causal)


def test_headline_flops():
    wl = workload_ragged64k()
    # causal, Lq == Lk: L(L+1)/2 visible pairs per head per sequence
    L = np.array(wl.lengths_q, dtype=np.int64)
    assert bench.visible_pairs(wl, True) == int((L * (L + 1) // 2).sum())
    assert abs(bench.algorithmic_flops(wl, True) / 1e9 - 2837.485) < 0.01
    assert bench.algorithmic_bytes(wl) == (3 * 65536 * 4096 * 2 + 65536 * 4096 * 2 + 4 * 65536 * 32)


def test_multi_gpu_request_is_refused(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "8"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
