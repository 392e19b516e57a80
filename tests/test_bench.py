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


def test_source_hash_ignores_comments_only():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\n\n  char q = \'"\';\n'
    assert bench.strip_comments(src) == 'int a = 1;\n const char* s = "x // y /* z */";\n  char q = \'"\';'
    assert bench.strip_comments("a/**/b") == "ab"
    # code changes show: one character of code differs
    assert bench.strip_comments("int a = 1;") != bench.strip_comments("int a = 2;")


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


def test_launch_stats():
    st = bench.launch_stats([0.25, 0.26, 0.24, 0.30])
    assert st["launches"] == 4
    assert st["mean_us"] == pytest.approx(262.5)
    assert st["median_us"] == pytest.approx(255.0)
    assert st["min_us"] == pytest.approx(240.0) and st["max_us"] == pytest.approx(300.0)


def test_full_parity_checks_every_element():
    # the CPU leg compares every element: one element off by more than the
    # tolerance anywhere in the output fails the check
    import numpy as np

    from exact_attention_52_amd import inputs
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS["c1_b1h2s128d64_fp16"]
    shape = (B, H, S, D, dtype, causal)
    words = inputs.gen_qkv(B, H, S, D, dtype, seed=0, qk_mult=mult)
    o_ref, l_ref, secs = bench.full_oracle(shape, words)
    assert secs >= 0 and o_ref.shape == (B, H, S, D)
    o_h = o_ref.astype(np.float16).astype(np.float32)  # a correctly rounded output
    l_h = l_ref.astype(np.float32)
    par = bench.parity_all(shape, o_h, l_h, o_ref, l_ref)
    assert par["ok"] and par["rows"] == B * H * S and par["elements_o"] == o_ref.size
    o_bad = o_h.copy()
    o_bad[B - 1, H - 1, S - 1, D - 1] += 3e-3
    assert not bench.parity_all(shape, o_bad, l_h, o_ref, l_ref)["ok"]
    l_bad = l_h.copy()
    l_bad[0, 1, 77] += 5e-3 * max(1.0, abs(float(l_h[0, 1, 77])))
    assert not bench.parity_all(shape, o_h, l_bad, o_ref, l_ref)["ok"]
    rate = bench.oracle_rate(shape, 2.0)
    assert rate["kind"] == "oracle" and rate["cores"] >= 1
    assert rate["value"] == pytest.approx(bench.flops(B, H, S, D, causal) / 2.0 / 1e12)


def test_roofline_bound_follows_the_workload():
    # B=2 H=16 S=4096 D=128: 2.75e11 FLOP at 2.5 PFLOP/s (110 us) against 134.7 MB at 8 TB/s (17 us): MFMA-bound
    r = bench.roofline((2, 16, 4096, 128, "fp16", False), 0.25)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(bench.flops(2, 16, 4096, 128, False) / 0.25e-3 / 1e12, rel=1e-5)
    # B=16 H=32 S=1024 D=64 causal: 6.87e10 FLOP (27.5 us) against 270.5 MB (33.8 us): HBM-bound
    r = bench.roofline((16, 32, 1024, 64, "fp16", True), 0.1)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] is None
    assert r["achieved"] == pytest.approx(bench.min_bytes(16, 32, 1024, 64) / 0.1e-3 / 1e9, rel=1e-3)
