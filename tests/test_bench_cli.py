"""bench.py's command-line contract, on the CPU: one GPU only, the workload
list, and the roofline traffic lookup from the committed summaries."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_list_names_the_headline_and_the_five_configurations():
    r = _run("--list")
    assert r.returncode == 0
    names = {line.split()[0]: int(line.split()[1]) for line in r.stdout.splitlines()}
    assert names["qmv_14336x4096_b4_g64_m1"] == 14336 * 4096 // 2 + 4 * 14336 * 64 + 2 * 4096 + 2 * 14336
    for w in ("tiny_qmv_256x512_b4_g64", "decode_qmv_4096x4096_b4_g64_m1", "decode_qmv_4096x4096_b4_g64_m4",
              "ffn_gate_up_14336x4096_b8_g64", "ffn_down_silu_resid_4096x14336_b8_g64",
              "moe_gather_64x2048x2048_b4_g64_t16_top8_unsorted",
              "moe_gather_64x2048x2048_b4_g64_t16_top8_sorted"):
        assert w in names
    for b in (2, 3, 5, 6, 8):
        for g in (32, 64, 128):
            assert f"qmv_14336x4096_b{b}_g{g}_m1" in names


def test_traffic_is_read_only_for_matching_sources():
    w = "qmv_14336x4096_b4_g64_m1"
    h = bench.kernel_source_hash(w)
    t = bench.read_traffic(w, h)
    if t is not None:                      # a summary taken on these sources
        assert 0.99 < t / bench.workloads()[w].nbytes < 1.2
    assert bench.read_traffic(w, "0" * 16) is None
    assert bench.read_traffic("no_such_workload", h) is None
