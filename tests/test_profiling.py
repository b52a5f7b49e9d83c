"""Host logic of the rocprofv3 summaries (no GPU): counter CSVs written here
by hand, in rocprofv3's column layout, go through the summarizers."""
import csv
import json
import os

from paged_kv_cache_364_amd import profiling

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
        "End_Timestamp"]


def write_pmc(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (kern, name, val, ns) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": name,
                        "Counter_Value": val, "Start_Timestamp": 1000, "End_Timestamp": 1000 + ns})


PF = "void pkv::prefill_kernel<128>(pkv::PrefillArgs)"
DM = "void pkv::decode_main<bf16_t, 128, 4>(pkv::DecodeArgs)"
CB = "void pkv::copy_blocks_kernel(pkv::CopyArgs)"


def test_traffic_summary_scales_by_calibration(tmp_path):
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    cal = 1 << 20
    # the copy reads cal bytes; FETCH_SIZE shows half of it, WRITE_SIZE all of it
    write_pmc(fd, [(CB, "FETCH_SIZE", cal / 2048, 10), (DM, "FETCH_SIZE", 100.0, 10), (DM, "FETCH_SIZE", 300.0, 10),
                   (DM, "FETCH_SIZE", 200.0, 10), ("other_kernel", "FETCH_SIZE", 5.0, 10)])
    write_pmc(wd, [(CB, "WRITE_SIZE", cal / 1024, 10), (DM, "WRITE_SIZE", 4.0, 10), (DM, "WRITE_SIZE", 4.0, 10),
                   (DM, "WRITE_SIZE", 4.0, 10)])
    out = str(tmp_path / "t.txt")
    r = profiling.traffic_summary(fd, wd, cal, out, "cmd")
    assert abs(r["scale_fetch"] - 2.0) < 1e-12 and abs(r["scale_write"] - 1.0) < 1e-12
    e = r["kernels"]["decode_main<bf16_t, 128, 4>"]
    assert e["fetch_kib"] == 200.0 and e["write_kib"] == 4.0  # medians
    assert abs(e["bytes"] - (200.0 * 1024 * 2 + 4.0 * 1024)) < 1e-6
    assert "other_kernel" not in json.dumps(r)
    back = profiling.read_traffic(out)
    assert profiling.traffic_bytes(back, ["decode_main<bf16_t, 128, 4>"]) == e["bytes"]
    # a figure whose kernel sources changed since is not reported
    back["kernels"]["decode_main<bf16_t, 128, 4>"]["sources_sha256"] = "0" * 64
    assert profiling.traffic_bytes(back, ["decode_main<bf16_t, 128, 4>"]) is None
    assert profiling.traffic_bytes(back, ["missing"]) is None


def test_traffic_calibration_is_the_first_copy(tmp_path):
    """Later copy_blocks dispatches (copy-on-write copies of a workload's
    setup) neither replace the calibration nor enter the table."""
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    cal = 1 << 20
    write_pmc(fd, [(CB, "FETCH_SIZE", cal / 2048, 10), (CB, "FETCH_SIZE", 7.0, 10), (DM, "FETCH_SIZE", 50.0, 10)])
    write_pmc(wd, [(CB, "WRITE_SIZE", cal / 1024, 10), (CB, "WRITE_SIZE", 7.0, 10), (DM, "WRITE_SIZE", 2.0, 10)])
    r = profiling.traffic_summary(fd, wd, cal, str(tmp_path / "t.txt"), "cmd")
    assert abs(r["scale_fetch"] - 2.0) < 1e-12 and abs(r["scale_write"] - 1.0) < 1e-12
    assert list(r["kernels"]) == ["decode_main<bf16_t, 128, 4>"]


def test_mfma_summary_medians(tmp_path):
    d = str(tmp_path / "m")
    write_pmc(d, [(PF, "MfmaUtil", 20.0, 300_000), (PF, "MfmaFlopsBF16", 1.9e11, 300_000),
                  (PF, "MfmaUtil", 24.0, 310_000), (PF, "MfmaFlopsBF16", 2.1e11, 310_000),
                  (PF, "MfmaUtil", 22.0, 305_000), (PF, "MfmaFlopsBF16", 2.0e11, 305_000),
                  (DM, "MfmaUtil", 0.0, 60_000), (DM, "MfmaFlopsBF16", 0.0, 60_000)])
    out = str(tmp_path / "m.txt")
    r = profiling.mfma_summary(d, out, "cmd")
    e = r["kernels"]["prefill_kernel<128>"]
    assert e["mfma_util_pct"] == 22.0 and e["bf16_flops"] == 2.0e11
    assert e["sources_sha256"] == profiling.sources_sha("prefill")
    assert r["kernels"]["decode_main<bf16_t, 128, 4>"]["mfma_util_pct"] == 0.0
    assert profiling.read_traffic(out)["kernels"]["prefill_kernel<128>"]["bf16_flops"] == 2.0e11
    text = open(out).read()
    assert text.startswith("# Matrix-core use") and "prefill_kernel<128>" in text
