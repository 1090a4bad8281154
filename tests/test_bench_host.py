"""Host checks of bench.py (no GPU): the one-GPU contract, the algorithmic
work it prices the roofline with, and the source check on profiled traffic."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_flops_of_the_layer_shape():
    # SMA: 4·N·P per visible (token, memory) pair, S·M(M-1)/2 pairs per
    # (batch, head): 4·128·64·256·(32·31/2)·4·32
    assert bench.sma_flops(bench.BASE) == 4 * 128 * 64 * 256 * 496 * 128
    assert bench.sma_flops(bench.BASE) / 1e9 == pytest.approx(532.576, abs=1e-3)
    # scan: per head 2·M·[S(S+1)/2·P + 2·S·N·P], per group 2·M·S(S+1)/2·N
    per_head = 2 * 32 * (256 * 257 / 2 * 64 + 2 * 256 * 128 * 64)
    per_group = 2 * 32 * 256 * 257 / 2 * 128
    assert bench.scan_flops(bench.BASE) == pytest.approx((per_head * 32 + per_group * 4) * 4)
    assert bench.scan_flops(bench.BASE) / 1e9 == pytest.approx(55.918, abs=1e-3)
    # the backward's SMA work: Zq/Zc once, dQ, dC and the two dΔH products
    assert bench.sma_bwd_flops(bench.BASE) == pytest.approx(3 * bench.sma_flops(bench.BASE))


def test_profiled_traffic_follows_the_source(tmp_path, monkeypatch):
    src, sha1, nbytes = bench.PROFILED_TRAFFIC["k_sma_grp"]
    path = os.path.join(bench.CSRC, src)
    with open(path, "rb") as f:
        live = hashlib.sha1(f.read()).hexdigest()
    assert bench.profiled_traffic("k_sma_grp") == (nbytes if live == sha1 else None)
    # a different source text: no figure
    (tmp_path / src).write_text("// changed\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.profiled_traffic("k_sma_grp") is None
