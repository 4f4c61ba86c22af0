"""The benchmark's host-side pieces run without a GPU: the CPU-baseline leg
(the fp64 oracle on a row sample), the byte and flop counts, and the
one-GPU guard."""

import subprocess
import sys
import os

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_leg():
    inp = synth.make_inputs("tiny_tree")
    r = bench.cpu_baseline(inp, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["cores"] >= 1
    assert r["one_thread"]["value"] > 0 and r["one_thread"]["unit"] == "GB/s"


def test_counts():
    inp = synth.make_inputs("tiny_tree")
    # 1 sequence, 1 KV head: (256 prefix + 8 draft) rows of K and V, D 64, fp32
    assert bench.kv_bytes(inp) == (256 + 8) * 2 * 64 * 4
    assert bench.step_flops(inp) > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
