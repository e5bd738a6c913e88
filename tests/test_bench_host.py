"""Host-side checks of the benchmark's arithmetic: the algorithmic bytes of a GEMM, the pages'
per-kernel floor, the confidence interval, and the counter summaries on synthetic rocprofv3
CSV files.  No GPU is used; summaries are written to a temporary folder."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench as B  # noqa: E402


def test_alg_bytes_of_the_gate_up_launch():
    # records 1.5 N K, bases N, pointers 4 (N + 1), escapes 4 E, X 2 M K, Y 4 M N
    n, k, m, e = 34816, 5120, 16, 29837
    parts = [267_386_880, 34_816, 139_268, 119_348, 163_840, 2_228_224]
    assert B.alg_bytes(n, k, m, e) == sum(parts) == 270_072_376


def test_byte_floor_takes_the_larger_bound():
    # M = 16: bytes at 90% of 8 TB/s dominate; M = 4096: FLOPs at 60% of 2.5 PFLOP/s dominate
    n, k = 34816, 5120
    t_bytes = B.alg_bytes(n, k, 16, 0) / (0.9 * 8000.0 * 1e3)
    assert B.byte_floor_us(n, k, 16, 0) == pytest.approx(t_bytes)
    t_flops = 2.0 * 4096 * n * k / (0.6 * 2500.0 * 1e6)
    assert B.byte_floor_us(n, k, 4096, 0) == pytest.approx(t_flops)
    assert t_flops > B.alg_bytes(n, k, 4096, 0) / (0.9 * 8000.0 * 1e3)


def test_ci95_of_known_samples():
    med, half = B.ci95([1.0, 2.0, 3.0, 4.0, 5.0])
    # t(0.975, 4) = 2.78; sample stdev of 1..5 = sqrt(2.5)
    assert med == 3.0
    assert half == pytest.approx(2.78 * 2.5 ** 0.5 / 5 ** 0.5)
    assert B.ci95([7.0]) == (7.0, None)


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_valu_arithmetic(tmp_path, monkeypatch):
    """Three launches per case in probe order; the middle one is summarised.  Counter rows are
    split over two dimensions (as rocprofv3 reports per shader engine) and must be summed."""
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    n, k = B.S.LAYER_SHAPES["gate_up"]
    rows, probe, disp = [], {}, 0
    for m in B.VALU_PROBE_M:
        for launch in range(3):
            disp += 1
            valu = 1_000_000 * m + launch
            for name, value in (("SQ_INSTS_VALU", valu + 200), ("SQ_INSTS_MFMA", 200), ("SQ_WAVES", 2048),
                                ("SQ_INSTS_SALU", 10), ("SQ_INSTS_LDS", 20), ("GRBM_GUI_ACTIVE", 8 * 1000)):
                for half in (0, 1):
                    rows.append({"Dispatch_Id": disp, "Kernel_Name": "void w12::k_gemm<...>",
                                 "Counter_Name": name, "Counter_Value": value / 2})
        probe[f"gate_up_M{m}"] = {"kernel": "k", "launch_us": [0.0, 50.0, 0.0], "grid": 512}
    pmc = tmp_path / "run_counter_collection.csv"
    _write_csv(pmc, rows)
    pj = tmp_path / "probe.json"
    pj.write_text("some log line\n" + json.dumps(probe) + "\n")
    B.summarize_valu(str(pmc), str(pj))
    out = json.loads((tmp_path / "profiles" / "gemm_gate_up_M1_M64_valu_counters.txt").read_text())
    assert out["budget_lane_ops_per_weight_at_6.4TBps"] == pytest.approx(1024 * 16 * 2.4e9 / (6.4e12 / 1.5), abs=0.01)
    for m in B.VALU_PROBE_M:
        c = out["launches"][f"gate_up_M{m}"]
        valu = 1_000_000 * m + 1   # the middle launch, MFMAs excluded
        assert c["valu_insts"] == valu and c["mfma_insts"] == 200 and c["waves"] == 2048
        assert c["valu_lane_ops_per_weight"] == pytest.approx(valu * 64 / (n * k), abs=1e-3)
        floor_us = valu * 4 / 1024 / 2.4e9 * 1e6
        assert c["valu_issue_floor_us"] == pytest.approx(floor_us, abs=0.01)
        assert c["valu_floor_over_time"] == pytest.approx(floor_us / 50.0, abs=1e-3)


def test_summarize_stalls_arithmetic(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rows, probe, disp = [], {}, 0
    for m in B.VALU_PROBE_M:
        for launch in range(3):
            disp += 1
            for name, value in (("SQ_WAVES", 1000), ("GRBM_GUI_ACTIVE", 8 * 5000), ("SQ_WAIT_ANY", 250_000),
                                ("SQ_WAIT_INST_ANY", 125_000), ("SQ_ACTIVE_INST_ANY", 1_000_000),
                                ("SQ_LDS_BANK_CONFLICT", 30), ("SQ_LDS_IDX_ACTIVE", 120), ("SQ_BUSY_CYCLES", 1)):
                rows.append({"Dispatch_Id": disp, "Kernel_Name": "void w12::k_gemm<...>",
                             "Counter_Name": name, "Counter_Value": value})
        probe[f"gate_up_M{m}"] = {"kernel": "k", "launch_us": [0.0, 40.0, 0.0], "grid": 256}
    pmc = tmp_path / "pmc.csv"
    _write_csv(pmc, rows)
    pj = tmp_path / "probe.json"
    pj.write_text(json.dumps(probe) + "\n")
    B.summarize_stalls(str(pmc), str(pj))
    out = json.loads((tmp_path / "profiles" / "gemm_gate_up_M1_M64_stall_counters.txt").read_text())
    c = out["launches"]["gate_up_M64"]
    # wave-cycles = 1000 waves x 5000 cycles; quad-cycle counters x 4
    assert c["kernel_cycles"] == 5000
    assert c["wait_any_frac"] == pytest.approx(4 * 250_000 / 5e6)
    assert c["wait_inst_issue_frac"] == pytest.approx(4 * 125_000 / 5e6)
    assert c["active_inst_frac"] == pytest.approx(1_000_000 / 5e6)
    assert c["lds_conflict_over_active"] == pytest.approx(0.25)


def test_kernel_names_match_the_instantiations():
    """The kernel names the benchmark reports are the ones rocprofv3 lists: the streaming kernel
    with its (Q pass, escape-window) flags, the window flag only where the path has that
    instantiation (GEMV M <= 4, 16-row tiles, wide tiles)."""
    gemv = {"path": 1, "m_tile": 1}
    assert B.kernel_name(gemv, 1) == "w12::k_gemm<w12::GemvPath<1>, false, false>"
    assert B.kernel_name(gemv, 2, dense=True) == "w12::k_gemm<w12::GemvPath<2>, false, true>"
    assert B.kernel_name(gemv, 6, dense=True) == "w12::k_gemm<w12::GemvPath<6>, false, false>"
    m16 = {"path": 2, "m_tile": 16}
    assert B.kernel_name(m16, 16) == "w12::k_gemm<w12::MfmaPath<1>, false, false>"
    assert B.kernel_name(m16, 9, dense=True) == "w12::k_gemm<w12::MfmaPath<1>, false, true>"
    m32 = {"path": 2, "m_tile": 32}
    assert B.kernel_name(m32, 32, dense=True) == "w12::k_gemm<w12::MfmaPath<2>, false, false>"
    wide = {"path": 3, "m_tile": 256}
    assert B.kernel_name(wide, 512) == "w12::k_gemm_wide<4, false, false>"
    assert B.kernel_name({"path": 3, "m_tile": 128}, 100, dense=True) == "w12::k_gemm_wide<2, false, true>"
