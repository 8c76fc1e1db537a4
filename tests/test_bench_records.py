"""Host logic of bench.py's counter records (no GPU): kernel names as the
records key them, and profiles/traffic.json / clock.json written from
rocprofv3 CSV output, on small synthetic CSVs."""
import csv
import json
import os

import pytest

import bench

HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
PF = ("void attn::(anonymous namespace)::prefill_bf16_kernel<128, true, true, false>"
      "(unsigned short const*, unsigned short const*, float*, int)")
ROPE = "attn::rope_bf16_kernel(unsigned short const*, unsigned short*, long long, int)"
COPY = "__amd_rocclr_copyBuffer"


def test_short_kernel_name():
    assert bench.short_kernel_name(PF) == "prefill_bf16_kernel<128, true, true, false>"
    assert bench.short_kernel_name(ROPE) == "rope_bf16_kernel"
    assert bench.short_kernel_name(COPY) == COPY
    # template arguments that hold parentheses stay whole
    assert bench.short_kernel_name("void attn::k<(anonymous namespace)::T, 4>(int)") == "k<T, 4>"


def _write(d, rows):
    """rows: (dispatch, kernel, grid, counter, value, start, end); a counter
    may repeat for one dispatch (one row per die)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEAD)
        for disp, name, grid, cn, cv, t0, t1 in rows:
            w.writerow([disp, disp, "Agent 1", 1, 1, 1, grid, 7, name, 256, 0, 0, 64, 0, 32, cn, cv, t0, t1])


def test_traffic_record(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    d = tmp_path / "cnt"
    # two dispatches of the kernel, FETCH_SIZE split over two rows each
    _write(d / "fetch", [(1, PF, 512, "FETCH_SIZE", 100.0, 0, 10), (1, PF, 512, "FETCH_SIZE", 50.0, 0, 10),
                         (2, PF, 512, "FETCH_SIZE", 200.0, 20, 30), (2, PF, 512, "FETCH_SIZE", 50.0, 20, 30),
                         (3, COPY, 64, "FETCH_SIZE", 1.0, 40, 41)])
    _write(d / "write", [(1, PF, 512, "WRITE_SIZE", 30.0, 0, 10), (2, PF, 512, "WRITE_SIZE", 50.0, 20, 30)])
    kib = (1 << 30) / 1024
    _write(d / "cal_fetch", [(1, COPY, 64, "FETCH_SIZE", kib / 2, 0, 10)])
    _write(d / "cal_write", [(1, COPY, 64, "WRITE_SIZE", kib, 0, 10)])
    bench.write_traffic_record(str(d))
    r = json.loads(rec.read_text())
    assert r["source_hash"] == bench.source_hash()
    assert r["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert r["calibration"]["write_factor"] == pytest.approx(1.0)
    k = r["kernels"]["prefill_bf16_kernel<128, true, true, false>"]
    assert k["fetch_kib"] == pytest.approx(200.0)   # mean of 150 and 250
    assert k["write_kib"] == pytest.approx(40.0)
    assert COPY not in r["kernels"]                 # no write pass for it, and runtime copies are dropped
    assert "extras" not in r
    # bench reads it back as bytes: fetch x 2 + write x 1, in bytes
    got = bench.recorded_traffic("prefill_bf16_kernel<128, true, true, false>")
    assert got == pytest.approx((200.0 * 2.0 + 40.0) * 1024)
    # a record taken on other sources is not used
    r["source_hash"] = "0" * 16
    rec.write_text(json.dumps(r))
    assert bench.recorded_traffic("prefill_bf16_kernel<128, true, true, false>") is None


def test_clock_record(tmp_path, monkeypatch):
    rec = tmp_path / "clock.json"
    monkeypatch.setattr(bench, "CLOCK_RECORD", str(rec))
    d = tmp_path / "clock"
    ns = 1_000_000  # 1 ms dispatch
    active = 2.0e6 * bench.XCDS  # 2e6 cycles per die over 1 ms -> 2 GHz
    busy = 0.5 * 2.0e6 * 1024     # half of the SIMD cycles busy on MFMA
    _write(d, [(1, PF, 512, "GRBM_GUI_ACTIVE", active, 0, ns),
               (1, PF, 512, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, ns),
               # a short dispatch is left out (its active count spills past it)
               (2, ROPE, 64, "GRBM_GUI_ACTIVE", 1e6, 2 * ns, 2 * ns + 20000),
               (2, ROPE, 64, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0, 2 * ns, 2 * ns + 20000)])
    bench.write_clock_record(str(d))
    r = json.loads(rec.read_text())
    k = r["kernels"]["prefill_bf16_kernel<128, true, true, false>"]
    assert k["sclk_ghz"] == pytest.approx(2.0)
    assert k["mfma_util_pct"] == pytest.approx(50.0)
    assert "rope_bf16_kernel" not in r["kernels"]
    assert bench.recorded_clock("prefill_bf16_kernel<128, true, true, false>") == pytest.approx(2.0)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = ('// header\n#include "x.h"\n/* block\n comment */\nint f(int a) {  // trailing\n'
           '    const char* s = "not // a comment"; return a + \'/\';\n}\n')
    (tmp_path / "k.hip").write_text(src)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.source_hash()
    (tmp_path / "k.hip").write_text(src.replace("// trailing", "// reworded").replace("block", "other"))
    assert bench.source_hash() == h0
    (tmp_path / "k.hip").write_text(src.replace("a + ", "a - "))
    assert bench.source_hash() != h0
    (tmp_path / "k.hip").write_text(src.replace("not // a", "not // b"))   # inside a string: code
    assert bench.source_hash() != h0
