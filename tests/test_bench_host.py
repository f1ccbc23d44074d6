"""Host logic of bench.py (no GPU): the counter-traffic records and their staleness check,
the oracle baseline workers, the one-GPU refusal."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows, 1):
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": i, "Correlation_Id": i, "Kernel_Name": name,
                                                  "Grid_Size": 256, "Counter_Name": counter, "Counter_Value": val})


def test_counter_summary_scales_by_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kernel, fname = bench.TRAFFIC["gqa_long"]
    dec = f"void lcd::{kernel}(lcd::DecodeParams)"
    other = "void lcd::decode_twopass_kernel<lcd::bf16_t, 128, 4, 0>(lcd::DecodeParams)"
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = (1 << 30) / 1024
    # fetch reads half the copied bytes, write all of them; a later copy of another size and
    # another decode instantiation are ignored
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [("fill", 1.0), (copy, gib_kib / 2), (copy, gib_kib / 2),
                                           (copy, gib_kib / 2), (dec, 1000.0), (dec, 1200.0), (copy, 7.0),
                                           (other, 9e9)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, gib_kib), (copy, gib_kib), (copy, gib_kib), (dec, 256.0),
                                           (dec, 256.0)])
    traffic = bench._counter_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "gqa_long")
    assert traffic == pytest.approx(1100.0 * 1024 * 2 + 256.0 * 1024)
    assert bench._traffic("gqa_long") == int(round(traffic))
    out = tmp_path / fname
    assert "--kernel-include-regex" in out.read_text()
    # a record taken on other sources is stale
    out.write_text(out.read_text().replace(bench._sources_digest(), "0" * 64))
    assert bench._traffic("gqa_long") is None
    assert bench._traffic("llama3_8b_layer") is None  # no record in tmp_path
    assert bench._traffic("tiny_streaming") is None  # no record kept for this workload


def test_counter_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    dec = f"void lcd::{bench.TRAFFIC['gqa_long'][0]}(lcd::DecodeParams)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(dec, 1000.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(dec, 1000.0)])
    with pytest.raises(SystemExit):
        bench._counter_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "gqa_long")


def test_snapkv_counter_summary_sums_the_kernels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = (1 << 30) / 1024
    rs = "void lcd::(anonymous namespace)::snapkv_rowstats_kernel<128, 1>(lcd::SnapkvParams)"
    ga = "lcd::(anonymous namespace)::snapkv_gather_kernel(lcd::SnapkvParams, int)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, gib_kib / 2)] * 3 + [(rs, 100.0), (rs, 300.0), (ga, 50.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, gib_kib)] * 3 + [(rs, 1.0), (rs, 1.0), (ga, 40.0)])
    total = bench._snapkv_counter_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    # per compress: the mean dispatch of each kernel, fetch scaled x2, write x1
    assert total == pytest.approx((200.0 + 50.0) * 1024 * 2 + (1.0 + 40.0) * 1024)
    text = (tmp_path / "snapkv_kernels_32k_traffic.md").read_text()
    assert "traffic-bytes-per-compress" in text and "snapkv_rowstats_kernel" in text


def test_mfma_summary_busy_fraction(tmp_path, monkeypatch):
    """busy / (1024 SIMDs x GRBM cycles / 8 XCDs), per scoring pass and window."""
    import csv

    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "m.csv"
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, name in ((1, "snapkv_rowstats_kernel<128, 4>"), (2, "snapkv_colscore_kernel<128, 4>")):
            for c, v in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0),
                         ("SQ_BUSY_CYCLES", 1.0), ("GRBM_GUI_ACTIVE", 8 * 1000.0)):
                wr.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=c, Counter_Value=v))
    bench._mfma_summary([f"128={path}"])
    text = (tmp_path / "snapkv_mfma_lobs_sweep.md").read_text()
    rows = [line for line in text.splitlines() if line.startswith("| 128 |")]
    assert len(rows) == 2 and all("| 0.5000 |" in r for r in rows)  # 500 busy of 1000 cycles
    assert all("| 0.410 |" in r for r in rows)  # ceiling 128 / 312


def test_oracle_workers_time_their_share():
    """The baseline workers run the oracle on disjoint shares and stop at their budget."""
    done0, el0 = bench._worker_streaming(("tiny_streaming", 0, 2, 100, 3, 10.0))
    done1, el1 = bench._worker_streaming(("tiny_streaming", 1, 2, 100, 3, 10.0))
    assert done0 + done1 == 3 and el0 > 0  # 1 slice per step, three steps, split two ways
    done, el = bench._worker_streaming(("tiny_streaming", 0, 1, 100, 50, 0.0))
    assert done == 0 and el == 0.0  # no budget: nothing timed
    assert 1 <= bench._oracle_cores() <= 16


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().out
