"""Host-side checks of bench.py (no GPU): the refusal of more than one GPU,
the lookup of measured HBM traffic in counter summaries (current and stale
kernel fingerprints), and the all-cores oracle baseline on a tiny sample."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _profiles(tmp_path, files):
    d = tmp_path / "profiles"
    d.mkdir()
    for name, text in files.items():
        (d / name).write_text(text)
    return str(tmp_path)


def test_measured_traffic_reads_current_summaries(tmp_path, monkeypatch):
    fp = bench.kernel_fingerprint()
    root = _profiles(tmp_path, {
        "fused_step_c2_x_pmc.md": f"kernel_fingerprint: {fp}\ntraffic_bytes_per_launch: 653000000\n",
        "fused_step_c3_c4_c5_pmc.md": (f"kernel_fingerprint: {fp}\ntraffic_bytes_per_step_c3: 5600000000\n"
                                       "traffic_bytes_per_step_c4: 18000000000\n"),
    })
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic("c2") == 653000000
    assert bench.measured_traffic("c3") == 5600000000
    assert bench.measured_traffic("c4") == 18000000000
    # no summary for these: no figure rather than another workload's
    assert bench.measured_traffic("c5") is None
    assert bench.measured_traffic("c1") is None


def test_measured_traffic_ignores_stale_summaries(tmp_path, monkeypatch):
    root = _profiles(tmp_path, {
        "fused_step_c2_x_pmc.md": "kernel_fingerprint: 0000000000000000\ntraffic_bytes_per_launch: 1\n",
        "fused_step_c3_c4_c5_pmc.md": "kernel_fingerprint: 0000000000000000\ntraffic_bytes_per_step_c4: 2\n",
    })
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic("c2") is None
    assert bench.measured_traffic("c4") is None


def test_per_launch_key_belongs_to_its_own_workload(tmp_path, monkeypatch):
    """A single-workload summary's traffic_bytes_per_launch applies to that
    workload only."""
    fp = bench.kernel_fingerprint()
    root = _profiles(tmp_path, {"fused_step_c2_x_pmc.md": f"kernel_fingerprint: {fp}\ntraffic_bytes_per_launch: 7\n"})
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic("c3") is None


@pytest.mark.timeout(120)
def test_all_cores_oracle_baseline_runs():
    from workloads import configs
    r = bench.cpu_baseline_all_cores(configs.ALL["c1"], 4096, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "elements/s"
    assert 1 <= r["cores"] <= 16
    assert r["value"] > 0 and r["gbs"] > 0


def test_memory_model_report_c4_prints_the_pages_table(capsys):
    """The bench line's config.memory_model at the 7.5B-parameter, Nd = 64
    workload: 120.0 / 31.4 / 16.6 / 1.9 GB, 2Psi = 1.5e10 and 3Psi =
    2.25e10 elements, from the library's zero_memory_model."""
    from workloads import configs
    from zero_partitioned_mixed_buffer_amd import binding as B
    mm = bench.memory_model_report(B, configs.C4)
    assert mm["psi"] == 7_500_000_000 and mm["nd"] == 64
    assert [r["stage"] for r in mm["stages"]] == ["DP", "Pos", "Pos+g", "Pos+g+p"]
    assert [r["total_gb_1dp"] for r in mm["stages"]] == [120.0, 31.4, 16.6, 1.9]
    assert [r["comm_elems"] for r in mm["stages"]] == [1.5e10, 1.5e10, 1.5e10, 2.25e10]
    assert mm["stages"][3]["reduction_vs_dp"] == 64.0
    bench.log_memory_model(mm)
    err = capsys.readouterr().err
    assert "DP 120.0 GB" in err and "Pos 31.4 GB" in err and "Pos+g 16.6 GB" in err and "Pos+g+p 1.9 GB" in err
    assert "2.25e+10 elements" in err and "1.5e+10 elements" in err


def test_host_cpu_reports_model_and_affinity():
    h = bench.host_cpu()
    assert h["affinity_cores"] >= 1 and h["host_cores"] >= h["affinity_cores"]
