"""Host-side pieces of bench.py (no GPU): the algorithmic byte counts, the counter-traffic
summary and its source-hash gate, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_algorithmic_bytes_at_the_headline_shape():
    # x, delta and y once each, B and C once per batch row and step, A once: bf16 except A
    w = workloads.WORKLOADS["m1p4b"]
    assert (w.Bt, w.L, w.D, w.N, w.io, w.dskip) == (4, 4096, 4096, 16, "bf16", False)
    xdy = 3 * 4 * 4096 * 4096 * 2
    bc = 2 * 4 * 4096 * 16 * 2
    a = 4096 * 16 * 4
    assert bench.alg_bytes_fwd(w) == xdy + bc + a == 403_963_904
    # the skip weight and the final states add their own bytes
    assert bench.alg_bytes_fwd(w.replace(dskip=True)) - bench.alg_bytes_fwd(w) == 4 * 4096
    assert bench.alg_bytes_fwd(w, last_state=True) - bench.alg_bytes_fwd(w) == 2 * 4 * 4096 * 16 * 4


def test_backward_algorithmic_bytes():
    # x, delta, dy in; dx, ddelta out (fp32 here); B, C in and dB, dC out; A in, dA out
    w = workloads.WORKLOADS["bwd"]
    s = 4
    want = 5 * w.Bt * w.L * w.D * s + 4 * w.Bt * w.L * w.N * s + 2 * w.D * w.N * 4
    assert bench.alg_bytes_bwd(w) == want


def _write_counters(path, counter, kernel_vals, copies):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for v in kernel_vals:
            wr.writerow({"Kernel_Name": "void msm::fwd_kernel<float, 2, 8>(msm::FwdArgs)",
                         "Grid_Size": 131072, "Counter_Name": counter, "Counter_Value": v})
        for grid, v in copies:
            wr.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": grid,
                         "Counter_Name": counter, "Counter_Value": v})
        # another counter in the same file is ignored
        wr.writerow({"Kernel_Name": "void msm::fwd_kernel<float, 2, 8>(msm::FwdArgs)",
                     "Grid_Size": 131072, "Counter_Name": "OTHER", "Counter_Value": 1e9})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the 256 MiB copy reads as 128 MiB of fetches (scale 2) and 256 MiB of writes (scale 1); a
    # small staging copy of the same kernel must not be taken for the calibration
    _write_counters(fetch, "FETCH_SIZE", [1000.0, 1002.0], [(4096, 7.0), (1 << 26, 131072.0)])
    _write_counters(write, "WRITE_SIZE", [500.0, 500.0], [(4096, 3.0), (1 << 26, 262144.0)])
    rec = bench.pmc_summary(str(fetch), str(write), "fwd_kernel", "unit", "cmd")
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (1001.0 * 2.0 + 500.0) * 1024
    assert rec["dispatches"] == [2, 2]
    with open(tmp_path / "profiles" / "traffic_unit.json") as f:
        assert json.load(f) == rec


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "selective_state_space_msm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel v1\n")
    (tmp_path / "profiles").mkdir()
    rec = {"source_hash": bench.source_hash(), "hbm_bytes_per_launch": 123.0}
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("x") == 123.0
    assert bench.measured_traffic("missing") is None
    (csrc / "k.hip").write_text("// kernel v2\n")
    assert bench.measured_traffic("x") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_valu_peak_follows_the_published_fp32_peak():
    # 157.3 TFLOP/s fp32 vector, halved for unpacked FP32 and halved for the two flops of an FMA:
    # the issue rate of 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz
    assert abs(bench.VALU_PEAK_TSLOTS - 157.3 / 4) < 1e-9
    assert abs(bench.VALU_PEAK_TSLOTS - 256 * 4 * 16 * 2.4e9 / 1e12) < 0.01
