"""Host-side checks of bench.py (no GPU): the one-GPU rule, the metric's
conventions, the keying of the committed traffic figures, and the CPU-baseline
object."""
import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_io_aware_13_amd import workloads as wl  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n, capsys):
    assert bench.main(["--gpus", str(n)]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_metric_conventions_at_the_bench_workload():
    w = wl.BY_KEY[wl.BENCH_KEY]
    assert (w.B, w.H, w.T, w.d, w.causal) == (1, 32, 8192, 128, True)
    # 4 B H T^2 d, halved for causal
    assert w.flops() == 4.0 * 32 * 8192 ** 2 * 128 / 2 == 549755813888.0
    # one read of Q, K, V and one write of O at 2 B/element, lse at 4 B/row
    assert w.algorithmic_bytes() == 4 * 32 * 8192 * 128 * 2 + 32 * 8192 * 4 == 269484032


def test_traffic_figure_is_keyed_to_the_kernel_source(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    fig = tmp_path / "t.json"
    fig.write_text(json.dumps({"kernel_sha256_16": bench.kernel_hash(str(src)), "workload": "c4",
                               "bytes_per_launch": 123}))
    assert bench.measured_traffic("c4", str(fig), str(src)) == 123
    assert bench.measured_traffic("c5", str(fig), str(src)) is None          # another workload
    src.write_text("// kernel, edited\n")
    assert bench.measured_traffic("c4", str(fig), str(src)) is None          # the source changed
    assert bench.measured_traffic("c4", str(tmp_path / "missing.json"), str(src)) is None


def test_traffic_files_are_named_by_workload_shape():
    assert bench.traffic_file(wl.BY_KEY["c4"]).endswith("profiles/fa_fwd_traffic_causal_b1h32t8192d128.json")
    assert bench.traffic_file(wl.BY_KEY["c3nc"]).endswith("fa_fwd_traffic_noncausal_b16h16t1024d64.json")
    assert bench.traffic_file(wl.BY_KEY["c4fp8"], "fa_fwd_fp8").endswith(
        "fa_fwd_fp8_traffic_causal_b1h32t8192d128.json")
    assert bench.profile_tag(wl.BY_KEY["decode"]) == "causal_b8hq32hkv8tq1tk32768d128"
    # every committed traffic figure names the workload its file name says
    for w in wl.WORKLOADS:
        for kernel in ("fa_fwd", "fa_fwd_fp8", "fa_bwd"):
            path = bench.traffic_file(w, kernel)
            if os.path.exists(path) and w.fp8 == (kernel == "fa_fwd_fp8"):
                with open(path) as f:
                    assert json.load(f)["workload"] == w.key, path


def test_variant_names_come_from_the_build():
    with pytest.raises(SystemExit):
        bench.main(["--variant", "nosuch"])


def test_cpu_baseline_object_on_the_small_workload():
    w = wl.BY_KEY["c1"]
    qb, kb, vb = wl.workload_inputs(w)
    r = bench.cpu_baseline(w, qb, kb, vb, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["cores"] >= 1 and np.isfinite(r["value"]) and r["value"] > 0
    assert "query rows" in r["sample"]


def test_committed_traffic_matches_the_current_kernel_sources():
    """The headline workload and the profiled companions carry a traffic figure:
    their committed counter runs were taken on the sources as they stand (a
    kernel source edited without new counter runs makes ``traffic`` null)."""
    cases = [("c4", "fa_fwd", bench.KERNEL_SRC), ("c2", "fa_fwd", bench.KERNEL_SRC),
             ("c3c", "fa_fwd", bench.KERNEL_SRC), ("c3nc", "fa_fwd", bench.KERNEL_SRC),
             ("c4fp8", "fa_fwd_fp8", bench.FP8_SRC), ("c4", "fa_bwd", bench.BWD_SRC)]
    for key, kernel, src in cases:
        path = bench.traffic_file(wl.BY_KEY[key], kernel)
        got = bench.measured_traffic(key, path, src)
        assert got is not None and got > wl.BY_KEY[key].algorithmic_bytes() * 0.9, (key, kernel, path)
