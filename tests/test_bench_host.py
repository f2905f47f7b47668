"""Host-side checks of the measurement harness (no GPU).

bench.py measures one GPU only and must refuse more; the committed rocprofv3
summaries must name the command that made them and, for the HBM counters,
carry every field bench.py reads.
"""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "single" in res.stderr
    assert res.stdout.strip() == ""  # no JSON line


def _summaries():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith(".txt"))


@pytest.mark.parametrize("name", _summaries())
def test_summary_names_its_command(name):
    text = open(os.path.join(PROFILES, name)).read()
    cmd = [line for line in text.splitlines() if line.startswith("command")]
    assert cmd, f"{name}: no command line"
    runs = [line for line in text.splitlines() if re.search(r"rocprofv3 --.* -- ", line)]
    assert runs, f"{name}: no rocprofv3 command"
    for line in runs:
        assert "bench.py" in line
    assert "_work" not in text  # only committed files are run


@pytest.mark.parametrize("name", [f for f in _summaries() if f.startswith("mfma_busy_")])
def test_mfma_summary_is_consistent(name):
    fields = {}
    for line in open(os.path.join(PROFILES, name)):
        m = re.match(r"^(\w+):\s*(\S+)$", line.strip())
        if m:
            fields[m.group(1)] = m.group(2)
    for key in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU",
                "SQ_INSTS_SALU", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "mfma_busy",
                "valu_bound_us_at_2400mhz", "mfma_bound_us_at_2400mhz", "source_digest"):
        assert key in fields, f"{name}: missing {key}"
    busy = float(fields["SQ_VALU_MFMA_BUSY_CYCLES"])
    # 8 XCDs, 1024 SIMDs
    assert float(fields["mfma_busy"]) == pytest.approx(
        busy / (float(fields["GRBM_GUI_ACTIVE"]) / 8 * 1024), abs=1e-4)
    # a 32x32x16 bf16 MFMA is 64 MOPs of 512 flops and keeps its SIMD busy 32 cycles
    mfma = float(fields["SQ_INSTS_MFMA"])
    assert busy == pytest.approx(32 * mfma, rel=0.02)
    assert float(fields["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) == pytest.approx(64 * mfma, rel=0.02)
    # the VALU issue bound: per-instruction costs spread over the 1024 SIMDs, at 2.4 GHz
    trans = float(fields["SQ_INSTS_VALU_TRANS_F32"])
    other = float(fields["SQ_INSTS_VALU"]) - mfma - trans
    cyc = (float(fields["valu_cost_trans_cycles"]) * trans
           + float(fields["valu_cost_other_cycles"]) * other) / 1024
    assert float(fields["valu_issue_cycles_per_simd"]) == pytest.approx(cyc, rel=1e-3)
    assert float(fields["valu_bound_us_at_2400mhz"]) == pytest.approx(cyc / 2400, rel=1e-3)


@pytest.mark.parametrize("name", [f for f in _summaries() if f.startswith("hbm_traffic_")])
def test_traffic_summary_is_consistent(name):
    fields = {}
    for line in open(os.path.join(PROFILES, name)):
        m = re.match(r"^(\w+):\s*(.+)$", line.strip())
        if m:
            fields[m.group(1)] = m.group(2)
    for key in ("fetch_factor", "write_factor", "kernel_fetch_kib_per_dispatch",
                "kernel_write_kib_per_dispatch", "fetch_bytes_per_launch",
                "write_bytes_per_launch", "traffic_bytes_per_launch", "source_digest"):
        assert key in fields, f"{name}: missing {key}"
    fetch_f, write_f = float(fields["fetch_factor"]), float(fields["write_factor"])
    # FETCH_SIZE counts half of a plain copy's reads on this chip, WRITE_SIZE all
    # of its writes; the calibration copy fixes both factors.
    assert 1.5 < fetch_f < 2.5 and 0.8 < write_f < 1.2
    # the per-launch figure is the median over the profiled dispatches
    fb = float(fields["kernel_fetch_kib_median"]) * 1024 * fetch_f
    wb = float(fields["kernel_write_kib_median"]) * 1024 * write_f
    for key in ("kernel_fetch_kib_per_dispatch", "kernel_write_kib_per_dispatch"):
        first = [float(x) for x in fields[key].split()]
        median = float(fields[key.replace("per_dispatch", "median")])
        assert all(abs(x - median) <= 0.05 * median for x in first), key
    # the factors are printed to 5 decimals: agree to 1e-5 relative
    assert fb == pytest.approx(float(fields["fetch_bytes_per_launch"]), rel=1e-5)
    assert wb == pytest.approx(float(fields["write_bytes_per_launch"]), rel=1e-5)
    assert float(fields["traffic_bytes_per_launch"]) == pytest.approx(
        float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"]), abs=2)


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_committed_fields_go_stale_with_the_sources(tmp_path, monkeypatch):
    """A counter summary counts only while the kernel sources are the ones it
    was taken with: another digest makes bench.py report null."""
    bench = _bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    text = ("mfma_busy: 0.5\nvalu_bound_us_at_2400mhz: 10.0\nmfma_bound_us_at_2400mhz: 20.0\n"
            "valu_non_mfma_insts: 1000\ntraffic_bytes_per_launch: 123\n")
    (tmp_path / "mfma_busy_w.txt").write_text(text + f"source_digest: {bench.kernel_source_digest()}\n")
    (tmp_path / "hbm_traffic_w.txt").write_text(text + "source_digest: 0000000000000000\n")
    assert bench.measured_mfma_busy("w") == 0.5
    assert bench.measured_traffic("w") is None          # stale digest
    assert bench.measured_mfma_busy("missing") is None  # no file


def test_valu_bound_ceilings(tmp_path, monkeypatch):
    """frac_ceiling_overlapped = flops / max(valu, mfma time) / peak and
    frac_ceiling_serial = flops / (valu + mfma time) / peak."""
    bench = _bench()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "mfma_busy_w.txt").write_text(
        "valu_bound_us_at_2400mhz: 30.0\nmfma_bound_us_at_2400mhz: 20.0\nvalu_non_mfma_insts: 7\n"
        f"source_digest: {bench.kernel_source_digest()}\n")
    peak = bench.PEAK_BF16_TFLOPS
    flops = 20e-6 * peak * 1e12  # exactly 20 us at the peak
    vb = bench.valu_bound("w", flops, peak)
    assert vb["valu_insts_per_launch"] == 7
    assert vb["frac_ceiling_overlapped"] == pytest.approx(20 / 30, abs=1e-4)
    assert vb["frac_ceiling_serial"] == pytest.approx(20 / 50, abs=1e-4)


def test_host_description_fields():
    d = _bench().host_description()
    assert set(d) == {"cpu_model", "affinity_cpus", "blas_threads"}
    assert d["affinity_cpus"] == len(os.sched_getaffinity(0))
