"""Host-side checks of bench.py (no GPU): a batch larger than the activations prepared
for it is refused before anything reaches the library, and the bench prepares enough
activation rows for every batch it is asked to time."""

import numpy as np
import pytest
import torch

import bench
import workloads as wl


def test_time_layer_refuses_a_batch_larger_than_its_activations():
    cfg = wl.CONFIGS["c3"]
    layer = {"x": torch.zeros((16, cfg.K), dtype=torch.float16)}
    with pytest.raises(ValueError, match="M=64"):
        bench.time_layer(cfg, 64, layer, 1, 0, sample_clocks=False)
    with pytest.raises(ValueError):
        bench.time_layer(cfg, 1, {"x": torch.zeros((1, cfg.K // 2), dtype=torch.float16)}, 1, 0,
                         sample_clocks=False)


def test_activations_cover_batches_beyond_the_configured_list():
    cfg = wl.CONFIGS["c3"]
    x = wl.activations(cfg, 64)
    assert x.shape == (64, cfg.K)
    np.testing.assert_array_equal(x[:16], wl.activations(cfg, 16))


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_takes_the_last_two_passes_of_the_headline_run(tmp_path, capsys):
    name = "_ZN5w4a1614gemv_m1_kernel" + bench.HEADLINE_KERNELS["c3:M1"][len("gemv_m1_kernel"):] + "Ev"
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows, t, d = [], 0, 0
    # 3 warm-up launches of 50 ns, 4 event-pair launches of 20 ns, 4 back-to-back of 10 ns,
    # then the same kernel on another grid (another layer), which must not join the run
    for dur in [50] * 3 + [20] * 4 + [10] * 4:
        d += 1
        rows.append([d, name, 131072, t, t + dur])
        t += dur
    rows.append([d + 1, name, 4096, t, t + 999])
    _write_csv(tmp_path / "trace" / "x_kernel_trace.csv", hdr, rows)
    bench.summarize_trace(str(tmp_path / "trace"), 4)
    out = capsys.readouterr().out
    assert "| event pairs | 4 | 0.02 |" in out
    assert "| back-to-back (timed region) | 4 | 0.01 |" in out
    assert "11 launches in the run" in out


def test_counter_means_skip_warm_up_and_sum_over_blocks(tmp_path):
    hdr = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    rows = []
    for d in range(1, 11):
        v = 1000.0 if d <= 5 else 10.0
        rows += [["gemm_big_kernel", d, "SQ_WAVES", v / 2], ["gemm_big_kernel", d, "SQ_WAVES", v / 2]]
    _write_csv(tmp_path / "p" / "pmc_counter_collection.csv", hdr, rows)
    per = bench._counter_rows(str(tmp_path / "p"))
    m, n = bench._means(per, "gemm_big_kernel")
    assert n == 5 and m["SQ_WAVES"] == 10.0
