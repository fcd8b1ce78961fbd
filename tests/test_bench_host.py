"""bench.py's host-side logic (no GPU): the one-GPU guard, the algorithmic byte
count, the committed HBM-traffic record, trace and counter summaries."""
import json
import os

import pytest

import bench
import workloads


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_algorithmic_kv_bytes_of_the_tiny_workload():
    # C1: one request, 512 context keys + 9 block keys, 2 kv-heads, head_dim 128, K and V
    # in bf16, every key visible to some query: (512 + 9) * 2 * 128 * 2 * 2 bytes
    assert bench.visible_kv_bytes(workloads.make("c1_tiny_d128", poison=False)) == 533504


def test_algorithmic_kv_bytes_count_only_the_window():
    # C4: causal, window 1024, block 16: the union of the block's windows is
    # (L + 15) - (L - 1023) + 1 = 1039 keys per request and kv-head
    wl = workloads.make("c4_causal_window_d256", poison=False)
    assert bench.visible_kv_bytes(wl) == wl.B * 1039 * wl.Hkv * wl.D * 2 * 2


def test_traffic_record_matches_the_kernel_sources():
    """The committed counter record must have been taken on the current attention
    sources; otherwise the bench line's traffic field would be null."""
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert rec["kernel_sha"] == bench.kernel_source_hash()
    assert bench.traffic_for(rec["kernel_sha"], 0) == rec["bytes_per_launch"]
    assert bench.traffic_for("0" * 16, 0) is None
    # the record's own arithmetic: counter KiB scaled by the known-size calibration runs
    assert rec["fetch_bytes_per_launch"] == pytest.approx(rec["fetch_kib_per_launch"] * 1024 *
                                                         rec["read_calibration"]["factor"])
    assert rec["write_bytes_per_launch"] == pytest.approx(rec["write_kib_per_launch"] * 1024 *
                                                         rec["write_calibration"]["factor"])
    assert rec["over_fetch_ratio"] == pytest.approx(rec["fetch_bytes_per_launch"] / rec["algorithmic_kv_bytes"])


def test_trace_summary_splits_phases_at_idle_gaps(tmp_path):
    path = tmp_path / "trace.csv"
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp",
            "k(args),0,10000", "k(args),20000,32000",            # phase 0: 10 and 12 us
            "k(args),10000000,10014000", "j(x),10020000,10021000"]  # phase 1 after a 10 ms gap
    path.write_text("\n".join(rows) + "\n")
    out = bench.summarize_trace(str(path))
    assert len(out["phases"]) == 2
    assert out["phases"][0]["kernels"]["k"]["count"] == 2
    assert out["phases"][0]["kernels"]["k"]["mean_us"] == pytest.approx(11.0)
    assert out["phases"][1]["kernels"]["k"]["median_us"] == pytest.approx(14.0)
    assert out["phases"][1]["kernels"]["j"]["count"] == 1


def test_counter_means_per_kernel(tmp_path):
    path = tmp_path / "pmc.csv"
    rows = ["Kernel_Name,Counter_Name,Counter_Value",
            "attn,FETCH_SIZE,100", "attn,FETCH_SIZE,300", "attn,WRITE_SIZE,7", "other,FETCH_SIZE,5"]
    path.write_text("\n".join(rows) + "\n")
    means = bench._pmc_means(str(path), "FETCH_SIZE")
    assert means["attn"] == pytest.approx(200.0)
    assert means["other"] == pytest.approx(5.0)


def test_timeline_summary_of_synthetic_stamps():
    import numpy as np

    # two calls, 16 workgroups (2 per XCD); stamps in 100 MHz ticks.  Workgroup w starts at
    # 10 + w ticks, spends 300 ticks (3 us) setting up, then tiles of 100 + 10 * (w // 2)
    # ticks (1 us, +0.1 us per XCD), 40 of them, then 400 ticks (4 us) of epilogue
    P, calls = 16, 2
    S = np.zeros((calls, P, 8), dtype=np.int64)
    for c in range(calls):
        for w in range(P):
            tile = 100 + 10 * (w // 2)
            S[c, w, 0] = 10 + w
            S[c, w, 1] = S[c, w, 0] + 300
            S[c, w, 2] = S[c, w, 1] + 40 * tile
            S[c, w, 3] = S[c, w, 2] + 400
            S[c, w, 4] = 40
    out = bench.summarize_timeline(S, np.array([100.0, 110.0]), tile_bytes=65536)
    assert out["setup_us"] == pytest.approx(3.0)
    assert out["epilogue_us"] == pytest.approx(4.0)
    assert out["per_xcd_per_tile_us"] == pytest.approx([1.0 + 0.1 * x for x in range(8)])
    assert out["per_tile_us"] == pytest.approx(1.35)  # median of the 16 workgroups' 1.0 .. 1.7
    ends = [(10 + w + 300 + 40 * (100 + 10 * (w // 2)) + 400 - 10) / 100 for w in range(P)]
    assert out["span_us"] == pytest.approx(max(ends))
    assert out["last_after_median_us"] == pytest.approx(max(ends) - np.median(ends))
    assert out["events_minus_span_us"] == pytest.approx(105.0 - max(ends))
    assert out["tiles_median"] == 40 and out["calls"] == 2
    assert out["loop_rate_gbps"] == pytest.approx(16 * 65536 / 1.35e-6 / 1e9)


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_settle_steps_bring_the_warm_up_to_the_floor():
    assert bench.SETTLE_STEPS >= 20
    assert os.path.exists(bench.TRAFFIC_FILE)
