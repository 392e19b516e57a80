"""The seeded input generator: known answers, determinism, slicing, moments,
rounding.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from exact_attention_52_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for case in kat["cases"]:
        ctr = [np.array([int(x, 16)], dtype=np.uint32) for x in case["ctr"]]
        key = [int(x, 16) for x in case["key"]]
        out = inputs.philox4x32_10(ctr, key)
        assert [f"{int(o[0]):08x}" for o in out] == case["out"]


def test_same_seed_same_bytes_and_streams_differ():
    a = inputs.gen_qkv(1, 2, 64, 64, "fp16", seed=0)
    b = inputs.gen_qkv(1, 2, 64, 64, "fp16", seed=0)
    c = inputs.gen_qkv(1, 2, 64, 64, "fp16", seed=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert not np.array_equal(a[0], a[1])  # Q and K streams differ
    assert not np.array_equal(a[1], a[2])


@pytest.mark.parametrize("start,n", [(0, 1), (1, 7), (3, 5), (4, 4), (1021, 37), (5, 0)])
def test_any_slice_regenerates(start, n):
    full = inputs.normals(7, 2, 2048)
    part = inputs.normals(7, 2, n, start=start)
    assert np.array_equal(full[start:start + n], part)


def test_moments():
    z = inputs.normals(0, 0, 1 << 20)
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    # fourth moment of N(0,1) is 3
    assert abs((z ** 4).mean() - 3.0) < 0.05
    assert np.all(np.isfinite(z))


def test_fp16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -2.5, 65504.0, 1e-8])
    words = inputs.round_to_bits(x, "fp16")
    ref = torch.tensor(x, dtype=torch.float64).to(torch.float16).view(torch.int16).numpy()
    assert np.array_equal(words.view(np.int16), ref)
    # ties go to even: 1 + 2^-11 sits halfway between 1 and 1 + 2^-10
    assert words[1] == 0x3C00 and words[2] == 0x3C02


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32).astype(np.float64)
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)])
    x = np.concatenate([x, ties])
    words = inputs.round_to_bits(x, "bf16")
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(words.view(np.int16), ref)
    assert words[-3] == 0x3F80 and words[-2] == 0x3F82


def test_peaky_multiplier_is_exact():
    z = inputs.normals(0, 0, 4096)
    w1 = inputs.round_to_bits(z, "fp16")
    w2 = inputs.round_to_bits(2.0 * z, "fp16")
    f1 = inputs.bits_to_float(w1, "fp16").astype(np.float64)
    f2 = inputs.bits_to_float(w2, "fp16").astype(np.float64)
    normal = np.abs(f1) > 2 ** -13  # away from the subnormal range
    assert np.array_equal(2 * f1[normal], f2[normal])


def test_workload_table():
    assert set(inputs.WORKLOADS) == {
        "c1_b1h2s128d64_fp16", "c2_b16h32s1024d64_fp16_causal",
        "c3_b4h16s2048d128_bf16_causal", "c4_b2h16s4096d128_fp16_peaky",
        "c5_b1h8s8192d256_bf16_causal"}
    assert inputs.WORKLOADS["c4_b2h16s4096d128_fp16_peaky"][-1] == 2.0
