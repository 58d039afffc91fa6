"""The seeded input generator: determinism, rounding and shapes (CPU)."""
import numpy as np

from ttt_workloads import (WORKLOADS, make_inputs, f64_to_bf16_bits, bf16_bits_to_f64, head_subset)


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0)
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0, 65504.0, 1e-40])
    b = f64_to_bf16_bits(x)
    back = bf16_bits_to_f64(b)
    assert back[0] == 1.0
    assert back[1] == 1.0
    assert back[2] == 1.0 + 2.0 ** -6          # tie rounds up to the even mantissa
    assert back[3] == -2.5
    assert back[4] == 0.0
    assert abs(back[5] - 65504.0) / 65504.0 < 2 ** -8


def test_bf16_rounding_error_bound():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000)
    y = bf16_bits_to_f64(f64_to_bf16_bits(x))
    assert np.max(np.abs(y - x) / np.abs(x)) <= 2.0 ** -8


def test_inputs_are_deterministic_and_exact():
    w = WORKLOADS["v4_momentum_4x8x2048_d128"].with_shape(B=1, H=2, T=70)
    a = make_inputs(w)
    b = make_inputs(w)
    assert np.array_equal(a.q_dev, b.q_dev) and np.array_equal(a.v_dev, b.v_dev)
    assert a.q_dev.dtype == np.uint16 and a.q_dev.shape == (1, 2, 70, 128)
    np.testing.assert_array_equal(bf16_bits_to_f64(a.k_dev), a.k64)
    # l2-normalised before rounding: norms within bf16 rounding of 1
    n = np.linalg.norm(a.q64, axis=-1)
    assert np.all(np.abs(n - 1.0) < 2e-2)


def test_softplus_and_swiglu_inputs():
    w = WORKLOADS["v2_swiglu_4x16x8192_d128_f512"].with_shape(B=1, H=2, T=10)
    x = make_inputs(w)
    assert x.a32.dtype == np.float32 and x.a32.shape == (1, 2, 10)
    assert x.w1_dev.shape == (2, 512, 128) and x.w3_64.shape == (2, 512, 128)
    assert abs(float(np.std(x.w1_64)) - 1 / np.sqrt(128)) < 0.01


def test_fp32_workload():
    w = WORKLOADS["v5_f32_1x1x256_d64"]
    x = make_inputs(w)
    assert x.q_dev.dtype == np.float32
    np.testing.assert_array_equal(x.q_dev.astype(np.float64), x.q64)


def test_head_subset():
    w = WORKLOADS["v3_softplus_8x16x4096_d128"]
    s = head_subset(w)
    assert len(s) == 8 and s[0] == 0 and s[-1] == w.B * w.H - 1
    assert s == head_subset(w)
