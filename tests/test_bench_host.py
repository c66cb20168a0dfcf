"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
workload options that select the measured configuration."""
import argparse
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _args(**kw):
    base = dict(config=2, focus=None, kv_dtype="bf16", rho=None, q_heads=None, steps=None)
    base.update(kw)
    return argparse.Namespace(**base)


def test_default_workload_is_the_128k_line():
    wl, K = bench.build_workload(_args())
    assert (wl.num_layers, wl.num_q_heads, wl.num_kv_heads, wl.head_dim) == (28, 16, 8, 128)
    assert wl.prefill == (131072,) and wl.batch == 1 and wl.rho == (0.125,)
    assert (wl.sink, wl.window, wl.block_size, wl.dtype) == (4, 2048, 16, "bf16")
    assert K == 1024


def test_workload_options():
    wl, _ = bench.build_workload(_args(kv_dtype="fp8", q_heads=32, rho=0.5, steps=64))
    assert wl.dtype == "fp8" and wl.num_q_heads == 32 and wl.rho == (0.5,)
    assert wl.name.endswith("_q32")
    wl4, K4 = bench.build_workload(_args(config=4, focus=0))
    assert wl4.focus is False and K4 == wl4.steps


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    h = bench.kernel_sha()
    assert len(h) == 16
    text = open(bench.KERNEL_SRC).read()
    commented = tmp_path / "commented.hip"
    commented.write_text("// a comment\n\n/* a block\n comment */\n" + text.replace("\n", "  // note\n", 3))
    changed = tmp_path / "changed.hip"
    changed.write_text(text + "\nint unused_symbol;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(commented))
    assert bench.kernel_sha() == h
    monkeypatch.setattr(bench, "KERNEL_SRC", str(changed))
    assert bench.kernel_sha() != h


def test_exact_rate_blocks_make_the_timed_rate_exact():
    """rho * (blocks * K) is whole for every K, so exactly rho of the timed steps fire."""
    import numpy as np

    from gated_kv_access_amd import workloads as W
    wl, _ = bench.build_workload(_args())
    for K, want in ((1024, 1), (20, 2), (5, 8), (8, 1), (12, 2), (1, 8)):
        r = bench.exact_rate_blocks(wl, K)
        assert r == want, (K, r)
        T = r * K
        fired = int((W.gen_scores(wl.with_(steps=T)) > 0).sum())
        assert fired == T // 8 and fired * 8 == T
    # Bernoulli draws (the other score modes) are timed in one block
    assert bench.exact_rate_blocks(W.config(1), 20) == 1
