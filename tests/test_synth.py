"""The seeded input generator: determinism, ranges and rounding (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def test_seed_determinism():
    a = synth.make_problem("bf16", 16, 24, 32, seed=3, ab_dist="normal", c_dist="zeros")
    b = synth.make_problem("bf16", 16, 24, 32, seed=3, ab_dist="normal", c_dist="zeros")
    c = synth.make_problem("bf16", 16, 24, 32, seed=4, ab_dist="normal", c_dist="zeros")
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B) and np.array_equal(a.C, b.C)
    assert not np.array_equal(a.A, c.A)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.float32([1.00390625, 1.01171875, -3.5e-39, 0.0, -0.0])])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_rounding_is_nearest():
    """Single rounding from the drawn double: no neighbouring fp16 value is closer.
    (torch goes through binary32 first and may differ by double rounding.)"""
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, 20000)
    ours = synth.f64_to_f16_bits(x)
    val = ours.view(np.float16).astype(np.float64)
    up = (ours.astype(np.int32) + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    dn = (ours.astype(np.int32) - 1).astype(np.uint16).view(np.float16).astype(np.float64)
    err = np.abs(val - x)
    assert np.all(err <= np.abs(up - x)) and np.all(err <= np.abs(dn - x))
    x32 = rng.uniform(-1, 1, 20000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f64_to_f16_bits(x32.astype(np.float64)), ref)


def test_shapes_and_layout_of_small_configs():
    p = synth.config_problem("C1")
    assert p.A.shape == (1, 256, 256) and p.A.dtype == np.uint16 and not p.a_col and not p.b_col
    vals = p.A.view(np.float16).astype(np.float64)
    assert vals.min() >= -1.0 and vals.max() <= 1.0 and abs(vals.mean()) < 0.01
    assert p.C.dtype == np.float32 and p.C.min() >= -1 and p.C.max() <= 1
    q = synth.config_problem("C4")
    assert q.batch == 8192 and q.A.shape == (8192, 64, 64) and q.C.shape == (8192, 64, 64)


def test_int8_ranges():
    p = synth.make_problem("i8", 64, 64, 4096, seed=3, c_range=(-(1 << 20), 1 << 20))
    assert p.A.min() == -128 and p.A.max() == 127
    assert p.C.dtype == np.int32 and p.C.min() >= -(1 << 20) and p.C.max() <= (1 << 20)


@pytest.mark.parametrize("name", ["C1", "C4"])
def test_exact_variant_is_small_integers(name):
    p = synth.exact_variant(name)
    vals = p.A.view(np.float16).astype(np.float64)
    assert set(np.unique(vals)).issubset({-1.0, 0.0, 1.0})
    assert np.all(p.C == np.round(p.C)) and np.abs(p.C).max() <= 8


def test_f64_problem_storage():
    p = synth.make_problem("f64", 5, 7, 9, b_col=True, pad=2, seed=9)
    assert p.A.dtype == np.float64 and p.B.dtype == np.float64 and p.C.dtype == np.float64
    assert p.A.shape == (1, 5, 11) and p.B.shape == (1, 7, 11) and p.C.shape == (1, 5, 9)
    assert p.A.min() >= -1 and p.A.max() < 1 and len(np.unique(p.A)) == p.A.size
    f = synth.make_problem("f64", 4, 4, 4, seed=9, ab_dist="small_int", c_dist="small_int",
                           c_range=(-8, 8))
    assert set(np.unique(f.A)) <= {-1.0, 0.0, 1.0} and np.all(f.C == np.round(f.C))
    q = synth.CONFIGS["F1"]
    assert (q["dtype"], q["M"], q["N"], q["K"]) == ("f64", 4096, 4096, 4096)
