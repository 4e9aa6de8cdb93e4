"""Host-side logic of bench.py that needs no GPU: the algorithmic byte
counts, and the kernel-source digest that ties profiles/ to the kernels."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_headline_call():
    """One rank's share of a 1 GiB, P = 8, INT4, fp32-state call: 20 + 3 pb -
    pb / P bytes per element with pb = 0.53125 (21.527 B, 11.557 GB)."""
    n, P = 536870912, 8
    alg = bench.algorithmic_bytes(P, n, 4, 4)
    pb = 0.5 + 4 / 128
    assert alg["k_quant_feedback"] == (P - 1) * (n // P) * (2 + 16 + pb)
    assert alg["k_owner_reduce_requant"] == (n // P) * (2 + 16 + P * pb)
    assert alg["k_dequant_gather"] == n * (pb + 2)
    assert abs(sum(alg.values()) / n - (20 + 3 * pb - pb / P)) < 1e-12
    assert round(sum(alg.values()) / 1e9, 3) == 11.557


def test_kernel_digest_does_not_depend_on_the_repository_location(tmp_path):
    """The same sources and flags give the same digest wherever the
    repository sits (the GPU machine runs it from another path)."""
    pkg = tmp_path / "error_compensated_bit_amd"
    shutil.copytree(os.path.join(ROOT, "error_compensated_bit_amd", "csrc"), pkg / "csrc")
    for f in ("__init__.py", "build.py"):
        shutil.copy(os.path.join(ROOT, "error_compensated_bit_amd", f), pkg / f)
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    out = subprocess.run([sys.executable, "-c", "import bench; print(bench.kernel_source_digest())"],
                         cwd=tmp_path, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == bench.kernel_source_digest()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr


def test_traffic_is_reported_only_for_a_profiled_configuration():
    """Each pmc summary in profiles/ covers one workload and launch
    configuration; a configuration no summary covers reports no traffic."""
    import glob
    import json
    import pytest
    found = 0
    for path in glob.glob(os.path.join(ROOT, "profiles", "pmc_*.json")):
        d = json.load(open(path))
        if d.get("kernel_source_digest") != bench.kernel_source_digest():
            continue
        cfg = {**bench.DEFAULT_CONFIG, **d["config"]}
        assert os.path.basename(path) == f"pmc_{bench.profile_key(d['workload'], cfg)}.json"
        t = bench.traffic_from_profile(d["workload"], "k_quant_feedback", cfg)
        assert t is not None
        found += 1
        for change in ({"group": 32}, {"rank": 5}, {"site": 77}):
            assert bench.traffic_from_profile(d["workload"], "k_quant_feedback", {**cfg, **change}) is None
    if not found:
        pytest.skip("no profile for the current kernel source")


def test_profile_key_names_only_non_default_settings():
    assert bench.profile_key("msg1gib_p8", dict(bench.DEFAULT_CONFIG)) == "msg1gib_p8"
    assert bench.profile_key("msg1gib_p8", {**bench.DEFAULT_CONFIG, "state": "bf16"}) == "msg1gib_p8_state-bf16"
    assert bench.profile_key("mixed_p8_16384x5120", {"site": 20}) == "mixed_p8_16384x5120_site-20"
    cmds = bench.profile_commands("mixed_p8_16384x5120", {"site": 20})
    assert all("--site 20" in c for k, c in cmds.items() if not k.startswith("copy"))
