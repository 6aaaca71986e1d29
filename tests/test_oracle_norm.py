"""Pins of the oracle's fused residual add + RMSNorm (the step that makes the
block's input; TensorFold issue #548, the CUDA claim of the shared layer
pieces: RMSNorm and the fused add + RMSNorm).

  r = h + residual (fp32 sum of two bf16 values), residual_out = bf16(r),
  x = r * gamma / sqrt(mean(r^2) + eps) in float64.

Checked against hand-rounded bf16 values, closed forms on constant, one-hot
and tiny rows, NumPy's vector norm on random rows, and exact invariance
under power-of-two scaling.
"""
import math

import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W

ONE = 0x3F80


def bits(v):
    return W.f32_to_bf16_bits(np.asarray(v, np.float32))


def val(b):
    return W.bf16_bits_to_f32(np.asarray(b, np.uint16)).astype(np.float64)


def run(h, res, gamma, eps=1e-5):
    h = None if h is None else np.asarray(h, np.uint16).reshape(1, -1)
    res = np.asarray(res, np.uint16).reshape(1, -1)
    r, x = oracle.add_rmsnorm(h, res, np.asarray(gamma, np.uint16), eps)
    return r[0], x[0]


def test_residual_is_the_bf16_of_the_sum_ties_to_even():
    H = 64
    g = np.full(H, ONE, np.uint16)
    cases = [  # (h, residual, expected residual_out bits)
        (1.0, 2.0 ** -8, 0x3F80),                    # 1 + 2^-8: a tie, to even (1.0)
        (1.0 + 2.0 ** -7, 2.0 ** -8, 0x3F82),        # 1 + 3 2^-8: a tie, to even (up)
        (1.0, 2.0 ** -8 + 2.0 ** -15, 0x3F81),       # just above the tie: up
        (3.5, -3.5, 0x0000),                         # exact cancellation: +0
        (-2.0, 0.5, 0xBFC0),                         # -1.5
        (2.0 ** 20, 1.0 + 2.0 ** -7, 0x4980),        # the small term vanishes
    ]
    for hv, rv, want in cases:
        r, _ = run(np.full(H, bits(hv)), np.full(H, bits(rv)), g)
        assert (r == want).all(), (hv, rv, hex(r[0]), hex(want))
    r, _ = run(None, np.full(H, bits(-1.5)), g)
    assert (r == 0xBFC0).all()


def test_constant_zero_and_tiny_rows_closed_form():
    H, eps = 128, 1e-5
    gamma = bits(np.linspace(0.5, 1.5, H))
    gv = val(gamma)
    for c in (1.0, -3.0, 0.15625):
        _, x = run(np.full(H, bits(c)), np.zeros(H, np.uint16), gamma, eps)
        assert np.allclose(x, gv * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    _, x = run(np.full(H, bits(2.0)), np.full(H, bits(-2.0)), gamma, eps)
    assert (x == 0.0).all()
    # tiny row: mean square 2^-20, comparable to eps
    _, x = run(None, np.full(H, bits(2.0 ** -10)), gamma, eps)
    assert np.allclose(x, gv * 2.0 ** -10 / math.sqrt(2.0 ** -20 + eps), rtol=1e-15, atol=0)


def test_one_hot_row_pins_the_mean_and_gamma_index():
    H, eps = 256, 1e-5
    gamma = np.full(H, ONE, np.uint16)
    gamma[36], gamma[37], gamma[38] = bits([0.25, 1.75, 0.5])
    res = np.zeros(H, np.uint16)
    res[37] = bits([3.0])[0]
    _, x = run(None, res, gamma, eps)
    want = 3.0 * val(gamma)[37] / math.sqrt(9.0 / H + eps)
    assert math.isclose(x[37], want, rel_tol=1e-15)
    assert (np.delete(x, 37) == 0.0).all()


@pytest.mark.parametrize("H", [64, 2048, 2688])
def test_random_rows_match_the_vector_norm(H):
    d = W.norm_inputs(16, H, seed=H)
    res_out, x = oracle.add_rmsnorm(d["h"], d["residual"], d["gamma"], d["eps"])
    r = val(d["h"]) + val(d["residual"])                 # exact in float64
    rms = np.linalg.norm(r, axis=1) / math.sqrt(H)
    want = r / np.sqrt(rms ** 2 + d["eps"])[:, None] * val(d["gamma"])[None, :]
    assert np.allclose(x, want, rtol=1e-6, atol=0)      # r itself is the fp32 sum
    assert (res_out == W.f32_to_bf16_bits(r.astype(np.float32))).all()


def test_power_of_two_scaling_is_exact_without_eps():
    d = W.norm_inputs(8, 512, seed=7, with_h=False)
    _, x = oracle.add_rmsnorm(None, d["residual"], d["gamma"], 0.0)
    scaled = W.f32_to_bf16_bits(val(d["residual"]).astype(np.float32) * np.float32(2.0 ** 12))
    _, x2 = oracle.add_rmsnorm(None, scaled, d["gamma"], 0.0)
    assert (x == x2).all()


def test_nan_stays_in_its_row():
    H = 64
    h = np.zeros((3, H), np.uint16)
    res = np.full((3, H), bits(1.0), np.uint16)
    h[1, 9] = W.BF16_NAN
    r, x = oracle.add_rmsnorm(h, res, np.full(H, ONE, np.uint16), 1e-5)
    assert r[1, 9] == W.BF16_NAN and (np.delete(r[1], 9) == ONE).all()
    assert np.isnan(x[1]).all() and np.isfinite(x[[0, 2]]).all()
