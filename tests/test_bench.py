"""CPU tests of bench.py's contract pieces (no GPU needed)."""
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
    assert r.stdout.strip() == ""


def test_flop_and_byte_conventions():
    # 4*B*H*S^2*D, halved when causal
    assert bench.flops(2, 16, 4096, 128, False) == 4.0 * 2 * 16 * 4096 ** 2 * 128
    assert bench.flops(4, 16, 2048, 128, True) == 2.0 * 4 * 16 * 2048 ** 2 * 128
    # Q, K, V read once + O written once (2 bytes each) + LSE (4 bytes per row)
    assert bench.min_bytes(2, 16, 4096, 128) == 8 * 2 * 16 * 4096 * 128 + 4 * 2 * 16 * 4096


def test_traffic_is_used_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic() is None  # no file
    f.write_text("# comment: ignored\nkernel_source_sha256_16: 0000000000000000\n"
                 "hbm_bytes_per_launch: 123456\n")
    assert bench.read_traffic() is None  # taken on another kernel source
    f.write_text(f"kernel_source_sha256_16: {bench.kernel_source_hash()}\nhbm_bytes_per_launch: 123456\n")
    assert bench.read_traffic() == pytest.approx(123456.0)


def test_backward_flop_convention():
    # five S x S x D GEMMs (2 flops per multiply-add), halved when causal; the
    # kernels execute seven (dQ recomputes S and dP)
    assert bench.bwd_flops(2, 16, 4096, 128, False) == 10.0 * 2 * 16 * 4096 ** 2 * 128
    assert bench.bwd_flops(2, 16, 4096, 128, True, gemms=7) == 7.0 * 2 * 16 * 4096 ** 2 * 128


def test_unfused_byte_convention():
    # the fused minimum plus S written and read in fp32, P written and read in
    # 16 bits, and the fp32 O and row factors written and read
    n = 2 * 16 * 4096
    assert bench.unfused_bytes(2, 16, 4096, 128) == (bench.min_bytes(2, 16, 4096, 128) + n * 4096 * 12
                                                     + n * 129 * 8)
