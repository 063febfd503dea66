"""bench.py's host-side arithmetic, without a GPU: the HBM-counter calibration
and traffic record, the SQ-counter derivations, the roofline entries, the
fractions of the achievable peaks and the step spread, each on small inputs
whose answers are worked out by hand."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]
TILE = "void msa::(anonymous namespace)::k_index_tile<__bf16, 128, 2, 16, false, true, false, 8>(msa::TileArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, counter, value, t0, t1 in rows:
            w.writerow({"Correlation_Id": disp, "Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1})


def test_pmc_calibration_and_traffic_record(tmp_path, monkeypatch, capsys):
    # A 1 GiB copy reads 1 GiB and writes 1 GiB; the counters read half of the
    # fetch (512 Ki KiB) and all of the write (1 Mi KiB): factors 2 and 1.
    # A small copy must not be taken for the calibration copy.
    f, w = str(tmp_path / "fetch"), str(tmp_path / "write")
    write_counters(f, [(1, COPY, "FETCH_SIZE", 524288, 0, 1), (2, COPY, "FETCH_SIZE", 512, 0, 1),
                       (3, TILE, "FETCH_SIZE", 1_000_000, 0, 1), (4, TILE, "FETCH_SIZE", 1_200_000, 0, 1)])
    write_counters(w, [(1, COPY, "WRITE_SIZE", 1048576, 0, 1), (2, COPY, "WRITE_SIZE", 1024, 0, 1),
                       (3, TILE, "WRITE_SIZE", 4000, 0, 1), (4, TILE, "WRITE_SIZE", 6000, 0, 1)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.summarize_pmc(f, w, "index_tile_topk", "unit_case")
    out = capsys.readouterr().out
    assert "FETCH_SIZE x 2.000, WRITE_SIZE x 1.000" in out
    rec = json.load(open(tmp_path / "index_tile_topk_unit_case_traffic.json"))
    # per launch: mean fetch 1.1e6 KiB x 1024 x 2 + mean write 5000 KiB x 1024 x 1
    assert rec["bytes_per_launch"] == pytest.approx(1.1e6 * 1024 * 2 + 5000 * 1024)
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["source_hash"] == bench.source_hash(bench.TRAFFIC_SOURCES["index_tile_topk"])


def test_sq_derivations(tmp_path, capsys):
    # 10 ms dispatches at 1.8 GHz on 8 XCDs; the matrix cores busy 75 % of the
    # cycles of 1024 SIMDs; 3200 VALU instructions (MFMA included) per 1000
    # MFMAs; half of the wave cycles waiting, 1 % on LDS; no bank conflicts.
    ns, act = 10_000_000, 1.8e7
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    rows_a, rows_b = [], []
    for disp in (1, 2):
        t0 = disp * 10 * ns
        for counter, value in (("GRBM_GUI_ACTIVE", 8 * act), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.75 * 1024 * act),
                               ("SQ_INSTS_MFMA", 1000), ("SQ_INSTS_VALU", 3200), ("SQ_WAVE_CYCLES", 1e9),
                               ("SQ_WAIT_INST_ANY", 5e8)):
            rows_a.append((disp, TILE, counter, value, t0, t0 + ns))
        for counter, value in (("SQ_WAIT_INST_LDS", 1e7), ("SQ_ACTIVE_INST_LDS", 100), ("SQ_LDS_BANK_CONFLICT", 0)):
            rows_b.append((disp, TILE, counter, value, t0, t0 + ns))
    write_counters(a, rows_a)
    write_counters(b, rows_b)
    bench.summarize_sq(a, b)
    row = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| k_index_tile")]
    assert row == ["| k_index_tile | 2 | 10.000 | 1.80 | 0.750 | 2.2 | 0.50 | 0.010 | 0.00 |"], row


def test_roofline_entries():
    r = bench.roofline("index_tile_topk", 23.27, flops=3.4907e13)
    assert r["bound"] == "mfma" and r["achieved"] == pytest.approx(3.4907e13 / 23.27e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0) and r["traffic"] is None
    h = bench.roofline("index_scan", 5.67, nbytes=34.36e9)
    assert h["bound"] == "hbm" and h["achieved"] == pytest.approx(34.36e9 / 5.67e-3 / 1e9)
    assert h["frac"] == pytest.approx(h["achieved"] / 8000.0)


def test_achievable_fractions_and_spread():
    line = {"roofline": {"bound": "mfma", "achieved": 1500.0},
            "legs": [{"index_scan": {"bound": "hbm", "achieved": 6000.0}}, {"other": {"bound": None}}]}
    bench.add_achievable(line, {"bf16_matmul_TFLOPs": 1400.0, "read_GBs": 6400.0})
    assert line["roofline"]["frac_of_achievable"] == pytest.approx(1500 / 1400)
    assert line["legs"][0]["index_scan"]["frac_of_achievable"] == pytest.approx(6000 / 6400)
    assert "frac_of_achievable" not in line["legs"][1]["other"]
    bench.add_achievable(line, None)  # probes skipped: nothing added, nothing raised
    assert bench.step_spread([3.0, 1.0, 2.0]) == {"min": 1.0, "median": 2.0, "max": 3.0, "steps": 3}
    assert bench.step_spread([]) is None
