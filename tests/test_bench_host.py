"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the traffic
summaries' lookup and its fingerprint guard."""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("wl,layer,tag", [("13b", "int8", "13b"), ("13b", "zeropoint", "13b-zeropoint"),
                                          ("decode1", "fp16w", "decode1-fp16w")])
def test_profile_tag(wl, layer, tag):
    assert bench.profile_tag(wl, layer) == tag


def test_traffic_is_read_only_for_matching_kernel_source(tmp_path, monkeypatch):
    fp = bench.kernel_fingerprint("tiled")
    p = tmp_path / "k_gemm_{}_traffic.txt"
    (tmp_path / "k_gemm_w_traffic.txt").write_text(
        f"# comment: 1\nkernel_fingerprint: {fp}\nworkload: w\nhbm_bytes_per_launch: 1234\n")
    (tmp_path / "k_gemm_v_traffic.txt").write_text(
        "kernel_fingerprint: 0000000000000000\nworkload: v\nhbm_bytes_per_launch: 99\n")
    (tmp_path / "k_gemm_u_traffic.txt").write_text(
        f"kernel_fingerprint: {fp}\nworkload: other\nhbm_bytes_per_launch: 5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.read_traffic("w") == 1234.0
    assert bench.read_traffic("v") is None          # taken on other kernel source
    assert bench.read_traffic("u") is None          # summary of another workload
    assert bench.read_traffic("missing") is None
    # a few-token workload's summary is keyed to the row-streaming kernel
    (tmp_path / "k_gemm_d_traffic.txt").write_text(
        f"kernel_fingerprint: {bench.kernel_fingerprint('gemv')}\nworkload: d\n"
        "hbm_bytes_per_launch: 7\n")
    assert bench.read_traffic("d", T=1) == 7.0
    assert bench.read_traffic("d", T=2048) is None


def test_committed_summaries_parse():
    # every committed traffic summary names its own workload and a byte count
    d = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(d) if n.endswith("_traffic.txt")]
    assert names
    for n in names:
        kv = {}
        for line in open(os.path.join(d, n)):
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
        assert kv["workload"] == n[len("k_gemm_"):-len("_traffic.txt")]
        assert float(kv["hbm_bytes_per_launch"]) > 0
