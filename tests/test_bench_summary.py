"""The benchmark's HBM-traffic summary (bench.pmc_summary) on synthetic
counter files: the calibration factor comes from the copy kernel, and the BF16
decode figure averages the forward-only burst's dispatches only. Those are the
launches whose algorithmic bytes the run reports. The split-form burst that
follows them and the passes before them are left out. CPU only."""
import csv
import json
import os

import bench

DEC = "void moe::dec_fused_kernel<false, 2, 8, 8, 1, false>(moe::DecArgs, moe::DecWsDev)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_decode_traffic_counts_the_forward_only_burst(tmp_path, monkeypatch):
    n = 4                                          # launches of the burst (roofline.launches)
    copy_kib = bench.COPY_BYTES / 1024.0
    # dispatch order: the copy, earlier passes, the burst, then the split burst (2 n shorter launches)
    fetch = [(COPY, 0.5 * copy_kib)] + [(DEC, 90.0)] * 6 + [(DEC, 200.0), (DEC, 202.0), (DEC, 198.0), (DEC, 200.0)] \
        + [(DEC, 40.0)] * (2 * n)
    write = [(COPY, 1.0 * copy_kib)] + [(DEC, 1.0)] * 6 + [(DEC, 3.0)] * n + [(DEC, 0.5)] * (2 * n)
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    run = {"metric": "m", "roofline": {"launches": n, "bytes_per_launch": 409600.0},
           "config": {"trace_steps": [8, 24]}}
    with open(tmp_path / "run.json", "w") as fh:
        fh.write(json.dumps(run) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    bench.pmc_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), str(tmp_path / "run.json"))
    out = json.load(open(tmp_path / "traffic.json"))
    dec = out["launches"]["decode_bf16_forward"]
    # FETCH_SIZE reads 0.5 KiB per KiB moved: the burst's mean 200 KiB is 400 KiB; WRITE_SIZE as is
    assert dec["bytes"] == round(200.0 * 1024 / 0.5 + 3.0 * 1024)
    assert dec["algorithmic_bytes"] == 409600.0
    assert out["calibration"]["bf16_run"]["FETCH_SIZE"]["counter_kib_per_true_kib"] == 0.5
    assert out["source_sha256"] == bench.forward_source_hash()
