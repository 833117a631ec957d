"""Host logic of bench.py, on the CPU: which traced kernels count as the timed
path, the counter calibration and per-launch HBM bytes, the clock / MFMA-busy
and duration summaries, the source-digest check that drops stale counter
figures, and the one-GPU refusal.  No GPU and no profiler are involved: the
inputs are small CSV files in rocprofv3's column layout."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FWD = "void fa::fwd_bf16_kernel<128, true, 8, 64, false>(__bf16 const*)"
FWD_SPLIT = "void fa::fwd_bf16_kernel<128, true, 1, 32, true>(__bf16 const*)"
FWD_256 = "void fa::fwd_bf16_kernel<256, true, 4, 32, false>(__bf16 const*)"
KV = "void fa::bwd_bf16_kernel<128, true, false>(__bf16 const*)"
KV_DROP = "void fa::bwd_bf16_dropout_kernel<128, true>(__bf16 const*)"
DQ = "void fa::bwd_dq_kernel<128, true, 8>(__bf16 const*)"
KV_DS = "void fa::bwd_bf16_ds_kernel<128, true>(__bf16 const*)"
DQ_DS = "void fa::bwd_dq_ds_kernel<128, true>(char const*)"
PRE = "_ZN2fa14bwd_pre_kernelILi128EDF16bEEvPKT0_S3_PKfPfS6_S6_mfiNS_9RowLayoutE"
PRE_256 = "_ZN2fa14bwd_pre_kernelILi256EDF16bEEvPKT0_S3_PKfPfS6_S6_mfiNS_9RowLayoutE"
COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16tofloat32_copy_kernel_cuda"
        "(at::TensorIteratorBase&)::{lambda(c10::BFloat16)#1}>(int)")


@pytest.mark.parametrize("name,short,want", [
    (FWD, "fwd_bf16_kernel", True), (FWD_SPLIT, "fwd_bf16_kernel", False), (FWD_256, "fwd_bf16_kernel", False),
    (KV, "bwd_bf16_kernel", True), (KV_DROP, "bwd_bf16_kernel", False), (DQ, "bwd_dq_kernel", True),
    (PRE, "bwd_pre_kernel", True), (PRE_256, "bwd_pre_kernel", False), (KV, "bwd_dq_kernel", False),
    (KV_DS, "bwd_bf16_ds_kernel", True), (KV_DS, "bwd_bf16_kernel", False), (DQ_DS, "bwd_dq_ds_kernel", True),
    (DQ_DS, "bwd_dq_kernel", False), (DQ, "bwd_dq_ds_kernel", False),
])
def test_headline_instance(name, short, want):
    assert bench._headline_instance(name, short) == want


FWD_DROP = "void fa::fwd_bf16_dropout_kernel<128, true, 8, 64>(__bf16 const*)"
KV_256 = "void fa::bwd256_kernel<true, false, true>(__bf16 const*)"


@pytest.mark.parametrize("name,key,want", [
    (FWD_DROP, "fwd_bf16_dropout_kernel", True), (FWD, "fwd_bf16_dropout_kernel", False),
    (KV_256, "bwd256_kernel_d256", True), (KV_DS, "bwd256_kernel_d256", False),
    ("void fa::bwd256_kernel<true, false, false>(__bf16 const*)", "bwd256_kernel_d256", False),
    ("void fa::bwd256_kernel<true, true, true>(__bf16 const*)", "bwd256_kernel_d256", False),
    ("void fa::bwd256_kernel<false, false, true>(__bf16 const*)", "bwd256_kernel_d256", False),
    ("void fa::bwd_dq_ds_kernel<256, true>(char const*)", "bwd_dq_ds_kernel_d256", True),
    (DQ_DS, "bwd_dq_ds_kernel_d256", False),
    ("void fa::fwd_fp8_kernel<128, true, 4, false>(unsigned char const*)", "fwd_fp8_kernel", True),
    ("void fa::fwd_fp8_kernel<128, true, 1, true>(unsigned char const*)", "fwd_fp8_kernel", False),
    ("void fa::fwd_fp8_kernel<128, true, 1, true>(unsigned char const*)", "fwd_fp8_kernel_split", True),
    (FWD_SPLIT, "fwd_bf16_kernel_split", True), (FWD, "fwd_bf16_kernel_split", False),
    ("void fa::fwd_merge_kernel<128>(float const*)", "fwd_merge_kernel", True),
    ("void fa::fwd_merge_kernel<64>(float const*)", "fwd_merge_kernel", False),
])

def test_detail_instance(name, key, want):
    assert bench._detail_instance(name, key) == want


def test_decode_traffic_is_split_plus_merge(tmp_path, monkeypatch):
    path = tmp_path / "c.json"
    dig = lambda k: bench.source_digest(bench.DETAIL_COUNTERS[k][1])
    json.dump({"fwd_bf16_kernel_split": {"hbm_bytes_per_launch": 1000, "source_digest": dig("fwd_bf16_kernel_split")},
               "fwd_merge_kernel": {"hbm_bytes_per_launch": 20, "source_digest": dig("fwd_merge_kernel")}},
              open(path, "w"))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    assert bench.decode_traffic("fwd_bf16_kernel_split") == 1020
    assert bench.decode_traffic("fwd_fp8_kernel_split") is None


def _write_pmc(path, rows):
    """rows: (dispatch, kernel, counter, value[, start, end])"""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            d, k, c, v = r[:4]
            s, e = (r[4], r[5]) if len(r) > 4 else (0, 1000)
            w.writerow([d, k, c, v, s, e])


def test_counter_summary_calibrates_on_the_copy_probe(tmp_path):
    """The probe copy reads copy_mib MiB and writes twice that; counters that
    read half the bytes are scaled by 2, and every kernel's bytes with the
    same factors (mean over its launches)."""
    mib = 16
    fetch = [(1, COPY, "FETCH_SIZE", mib * 1024 / 2), (2, FWD, "FETCH_SIZE", 1000.0), (3, FWD, "FETCH_SIZE", 3000.0),
             (4, FWD_256, "FETCH_SIZE", 9e9), (5, KV, "FETCH_SIZE", 500.0), (6, KV_256, "FETCH_SIZE", 700.0),
             (7, FWD_DROP, "FETCH_SIZE", 80.0)]
    write = [(1, COPY, "WRITE_SIZE", 2 * mib * 1024), (2, FWD, "WRITE_SIZE", 100.0), (3, FWD, "WRITE_SIZE", 300.0),
             (4, FWD_256, "WRITE_SIZE", 9e9), (5, KV, "WRITE_SIZE", 50.0), (6, KV_256, "WRITE_SIZE", 70.0),
             (7, FWD_DROP, "WRITE_SIZE", 8.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "c.json"
    _write_pmc(fp, fetch)
    _write_pmc(wp, write)
    bench.summarize_counters(str(fp), str(wp), mib, str(out))
    c = json.load(open(out))
    assert c["copy_probe"]["fetch_factor"] == pytest.approx(2.0)
    assert c["copy_probe"]["write_factor"] == pytest.approx(1.0)
    assert c["fwd_bf16_kernel"]["fetch_kib_per_launch"] == pytest.approx(2000.0)
    assert c["fwd_bf16_kernel"]["hbm_bytes_per_launch"] == int((2000.0 * 2 + 200.0) * 1024)
    assert c["bwd_bf16_kernel"]["hbm_bytes_per_launch"] == int((500.0 * 2 + 50.0) * 1024)
    assert c["fwd_bf16_kernel"]["source_digest"] == bench.source_digest(bench.KERNEL_SOURCES["fwd_bf16_kernel"])
    assert "bwd_dq_kernel" not in c
    assert c["bwd256_kernel_d256"]["hbm_bytes_per_launch"] == int((700.0 * 2 + 70.0) * 1024)
    assert c["fwd_bf16_dropout_kernel"]["hbm_bytes_per_launch"] == int((80.0 * 2 + 8.0) * 1024)
    assert c["bwd256_kernel_d256"]["source_digest"] == bench.source_digest(
        bench.DETAIL_COUNTERS["bwd256_kernel_d256"][1])


def test_traffic_is_dropped_once_the_sources_change(tmp_path, monkeypatch):
    path = tmp_path / "c.json"
    good = bench.source_digest(bench.KERNEL_SOURCES["bwd_bf16_kernel"])
    json.dump({"bwd_bf16_kernel": {"hbm_bytes_per_launch": 123, "source_digest": good},
               "bwd_dq_kernel": {"hbm_bytes_per_launch": 456, "source_digest": "0000000000000000"}},
              open(path, "w"))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    assert bench.traffic_from_counters("bwd_bf16_kernel") == 123
    assert bench.traffic_from_counters("bwd_dq_kernel") is None
    assert bench.traffic_from_counters("fwd_bf16_kernel") is None


def test_busy_summary_clock_and_fraction(tmp_path, capsys):
    """GRBM_GUI_ACTIVE sums 8 XCDs; a 500 us dispatch with 8 * 1e6 active
    cycles ran at 2 GHz, and 0.5 * 1e6 * 1024 busy cycles are half of every
    SIMD's cycles."""
    rows = []
    for d in range(3):
        rows.append((d, KV, "GRBM_GUI_ACTIVE", 8e6, 0, 500_000))
        rows.append((d, KV, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5e6 * 1024, 0, 500_000))
    p = tmp_path / "b.csv"
    _write_pmc(p, rows)
    bench.summarize_busy(str(p), 3)
    out = capsys.readouterr().out
    line = next(l for l in out.splitlines() if "bwd_bf16_kernel" in l)
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "3" and cells[2] == "500.0" and cells[3] == "2.00" and cells[4] == "0.500"


def test_stall_summary_counts_and_fractions(tmp_path, capsys):
    """Two passes over the same two dispatches: per wave 100000 VALU
    instructions besides 20000 MFMA ones; 8 XCDs x 1e6 active cycles are
    1e6 cycles of each of the 1024 SIMDs, of which 4 x 1e5 x 1024 (0.4) are
    VALU issue and 0.5e6 x 1024 matrix-pipe busy; the wave-cycle fractions
    are taken as given."""
    a, b = [], []
    for dsp in range(2):
        for name, val in (("SQ_WAVE_CYCLES", 1000.0), ("SQ_BUSY_CYCLES", 1.0), ("SQ_WAIT_INST_ANY", 300.0),
                          ("SQ_ACTIVE_INST_ANY", 450.0), ("SQ_ACTIVE_INST_VALU", 1.0), ("SQ_ACTIVE_INST_LDS", 1.0),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5e6 * 1024), ("SQ_WAIT_ANY", 250.0)):
            a.append((dsp, KV, name, val, 0, 1))
        for name, val in (("SQ_INSTS_VALU", 120000.0 * 1024), ("SQ_INSTS_MFMA", 20000.0 * 1024),
                          ("SQ_INSTS_LDS", 30000.0 * 1024), ("SQ_INSTS_SALU", 1.0), ("SQ_ACTIVE_INST_MISC", 1.0),
                          ("SQ_WAVES", 1024.0), ("GRBM_GUI_ACTIVE", 8e6)):
            b.append((dsp, KV, name, val, 0, 1))
    pa, pb = tmp_path / "a.csv", tmp_path / "b.csv"
    _write_pmc(pa, a)
    _write_pmc(pb, b)
    bench.summarize_stalls(str(pa), str(pb), 2)
    line = next(l for l in capsys.readouterr().out.splitlines() if "bwd_bf16_kernel" in l)
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1:] == ["1024", "100000", "20000", "30000", "0.40", "0.50", "0.45", "0.30", "0.25"], cells


def test_trace_summary_last_launches(tmp_path, capsys):
    p = tmp_path / "t.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, us in enumerate([900, 100, 200, 300]):
            w.writerow([DQ, i * 10_000_000, i * 10_000_000 + us * 1000])
    bench.summarize_trace(str(p), 2)
    line = next(l for l in capsys.readouterr().out.splitlines() if "bwd_dq_kernel" in l)
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "4" and cells[2] == "375.0" and cells[3] == "250.0" and cells[4] == "100.0"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ds_buffer_bytes_and_backward_kernels():
    """The dS buffer the hand-off's dQ kernel reads (4 KB per 64-query x
    32-key slice; causal: 2i + 2 slices for query block i) and the work each
    backward kernel is credited with per method."""
    assert bench.ds_buffer_bytes(1, 32, 8192, True) == 32 * 4096 * 128 * 129
    assert bench.ds_buffer_bytes(4, 16, 1024, False) == 64 * 4096 * 16 * 32
    assert bench.ds_buffer_bytes(1, 1, 100, True) == 4096 * 2 * 3
    # within 1% of 2 bytes per kept (query, key) pair at the headline shape
    pairs = 32 * 8192 * 8193 // 2
    assert abs(bench.ds_buffer_bytes(1, 32, 8192, True) / (2 * pairs) - 1) < 0.01
    k = bench.backward_kernels("handoff", 10.0, 1000, 5000, 1.0, 0.5)
    assert k == [("bwd_bf16_ds_kernel", 1.0, "mfma", 40.0), ("bwd_dq_ds_kernel", 0.5, "hbm", 5000 + 4000)]
    k = bench.backward_kernels("recompute", 10.0, 1000, 5000, 1.0, 0.5)
    assert k == [("bwd_bf16_kernel", 1.0, "mfma", 40.0), ("bwd_dq_kernel", 0.5, "mfma", 30.0)]
    k = bench.backward_kernels("atomic", 10.0, 1000, 5000, 1.0, 0.5)
    assert k[0] == ("bwd_bf16_kernel", 1.0, "mfma", 50.0) and k[1][2] == "hbm"
