"""Pins of the oracle's NVFP4 experts (TensorFold issue #548, the core/quant
split: ModelOpt NVFP4 with uint8 [N, K/2] codes, an e4m3 scale every 16
inputs and a global scale; the float64 reference decoders).

* E2M1 values written out by hand for all 16 codes (sign bit 3, exponent
  bits 2..1 with bias 1, mantissa bit 0; no infinities or NaN), -0 kept.
* The packing: element c in byte c // 2, low nibble first.
* A hand layer whose one routed path is worked out by hand: up weight
  3.0 x scale 1.0 x global 0.5 = 1.5, relu^2 2.25, down weight
  1.0 x 2.0 x 0.25 = 0.5, output 1.125 times the routing weight.
* A layer against a dense float64 NumPy computation whose decode is written
  independently (a table of the eight magnitudes, NumPy nibble extraction,
  the E4M3 decode pinned in test_oracle_fp8.py).
"""
import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W

HAND = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_hand_values():
    # codes 0..15, two per byte, low nibble first
    packed = np.array([(2 * i) | ((2 * i + 1) << 4) for i in range(8)], np.uint8)
    got = oracle.fp4_decode(packed, 16)
    assert got.tolist() == HAND
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_packing_is_low_nibble_first():
    assert oracle.fp4_decode(np.array([0x21, 0xF8], np.uint8), 4).tolist() == [0.5, 1.0, -0.0, -6.0]
    assert oracle.fp4_decode(np.array([0x7A], np.uint8), 1).tolist() == [-1.0]


def _hand_layer():
    H = I = 64
    wl = W.Workload("pin_nvfp4", T=2, H=H, I=I, E=2, k=1, act="relu2", wfmt="nvfp4",
                    norm_topk=False)
    x = np.zeros((2, H), np.float32)
    x[:, 0] = 1.0
    router = np.zeros((2, H), np.float32)
    router[1, 0] = -1.0                           # expert 0 wins, weight sigmoid(0) = 1/2
    w_up = np.zeros((2, I, H // 2), np.uint8)
    w_down = np.zeros((2, H, I // 2), np.uint8)
    up_sc = np.full((2, I, H // 16), 0x38, np.uint8)    # e4m3 1.0
    down_sc = np.full((2, H, I // 16), 0x38, np.uint8)
    w_up[0, 0, 0] = 0x05                          # element 0 of up row 0: 3.0
    down_sc[0, 0, 0] = 0x40                       # e4m3 2.0 for down row 0, inputs 0..15
    w_down[0, 0, 0] = 0x02                        # element 0 of down row 0: 1.0
    inp = {"x": W.f32_to_bf16_bits(x), "router_w": router, "bias": np.zeros(2, np.float32),
           "w_up": w_up, "w_down": w_down, "w_up_scales": up_sc, "w_down_scales": down_sc,
           "w_up_global": np.array([0.5, 1.0], np.float32),
           "w_down_global": np.array([0.25, 1.0], np.float32)}
    return wl, inp


def test_hand_layer():
    wl, inp = _hand_layer()
    out, ids, w = oracle.forward_tokens(wl, inp, np.arange(2), want_routing=True)
    assert (ids == 0).all() and (w == 0.5).all()
    expect = np.zeros((2, wl.H))
    expect[:, 0] = 0.5 * 0.5 * 1.5 ** 2           # w x down weight x relu^2(1.5)
    assert (out == expect).all()


def _np_fp4(packed, n_cols):
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    lo, hi = packed & 15, packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], n_cols)
    v = mag[codes & 7]
    return np.where(codes & 8, -v, v)


@pytest.mark.parametrize("name", ["mid_nvfp4", "mid_nvfp4_relu2"])
def test_nvfp4_layer_matches_dense_float64(name):
    wl = W.by_name(name)
    inp = W.generate(wl)
    toks = np.arange(12)
    out, ids, w = oracle.forward_tokens(wl, inp, toks, want_routing=True)

    def dense(codes, scales, g):
        E, N, K2 = codes.shape
        v = _np_fp4(codes, 2 * K2)
        s = oracle.fp8_decode(scales.reshape(-1)).reshape(scales.shape)
        return v * np.repeat(s, 16, axis=2) * g.astype(np.float64)[:, None, None]

    wu = dense(inp["w_up"], inp["w_up_scales"], inp["w_up_global"])
    wd = dense(inp["w_down"], inp["w_down_scales"], inp["w_down_global"])
    x = W.bf16_bits_to_f32(inp["x"][toks]).astype(np.float64)

    def act(p, n):
        if wl.act == "swiglu":
            g, u = p[:n], p[n:]
            return g / (1.0 + np.exp(-g)) * u
        r = np.where(p < 0, 0.0, p)
        return r * r

    ref = np.zeros((toks.size, wl.H))
    for i in range(toks.size):
        for j in range(wl.k):
            e = ids[i, j]
            ref[i] += w[i, j] * (wd[e] @ act(wu[e] @ x[i], wl.I))
        ref[i] *= wl.rsf
        if wl.I_shared:
            su = W.bf16_bits_to_f32(inp["shared_up"]).astype(np.float64)
            sd = W.bf16_bits_to_f32(inp["shared_down"]).astype(np.float64)
            ref[i] += sd @ act(su @ x[i], wl.I_shared)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- MXFP4
# OCP MX: the same E2M1 codes with an E8M0 scale every 32 inputs,
# 2^(b - 127), 0xFF NaN, and no global scale.

def test_e8m0_hand_values():
    got = oracle.e8m0_decode(np.array([127, 128, 120, 1, 0, 254, 255], np.uint8))
    assert got[:6].tolist() == [1.0, 2.0, 2.0 ** -7, 2.0 ** -126, 2.0 ** -127, 2.0 ** 127]
    assert np.isnan(got[6])


def test_mxfp4_hand_layer():
    H = I = 64
    wl = W.Workload("pin_mxfp4", T=2, H=H, I=I, E=2, k=1, act="relu2", wfmt="mxfp4",
                    norm_topk=False)
    x = np.zeros((2, H), np.float32)
    x[:, 0] = 1.0
    router = np.zeros((2, H), np.float32)
    router[1, 0] = -1.0
    w_up = np.zeros((2, I, H // 2), np.uint8)
    w_down = np.zeros((2, H, I // 2), np.uint8)
    up_sc = np.full((2, I, H // 32), 127, np.uint8)
    down_sc = np.full((2, H, I // 32), 127, np.uint8)
    w_up[0, 0, 0] = 0x05                          # 3.0
    up_sc[0, 0, 0] = 126                          # x 1/2 = 1.5; relu^2 2.25
    w_down[0, 0, 0] = 0x02                        # 1.0
    down_sc[0, 0, 0] = 125                        # x 1/4
    down_sc[0, 0, 1] = 255                        # NaN scale on inputs 32..63 of down row 0
    up_sc[0, 1, 1] = 255                          # and on up row 1, inputs 32..63
    inp = {"x": W.f32_to_bf16_bits(x), "router_w": router, "bias": np.zeros(2, np.float32),
           "w_up": w_up, "w_down": w_down, "w_up_scales": up_sc, "w_down_scales": down_sc}
    out = oracle.forward_tokens(wl, inp, np.arange(2))
    # up row 1 is NaN (NaN scale x 0 codes), so down row 0 and every other
    # down row meet a NaN activation: every output is NaN ...
    assert np.isnan(out).all()
    # ... and without the NaN scales the one path is worked out by hand
    up_sc[0, 1, 1] = 127
    down_sc[0, 0, 1] = 127
    out = oracle.forward_tokens(wl, inp, np.arange(2))
    expect = np.zeros((2, wl.H))
    expect[:, 0] = 0.5 * 0.25 * 1.5 ** 2
    assert (out == expect).all()


@pytest.mark.parametrize("name", ["mid_mxfp4", "mid_mxfp4_relu2"])
def test_mxfp4_layer_matches_dense_float64(name):
    wl = W.by_name(name)
    inp = W.generate(wl)
    toks = np.arange(12)
    out, ids, w = oracle.forward_tokens(wl, inp, toks, want_routing=True)

    def dense(codes, scales):
        v = _np_fp4(codes, 2 * codes.shape[2])
        s = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
        return v * np.repeat(s, 32, axis=2)

    wu = dense(inp["w_up"], inp["w_up_scales"])
    wd = dense(inp["w_down"], inp["w_down_scales"])
    x = W.bf16_bits_to_f32(inp["x"][toks]).astype(np.float64)

    def act(p, n):
        if wl.act == "swiglu":
            g, u = p[:n], p[n:]
            return g / (1.0 + np.exp(-g)) * u
        r = np.where(p < 0, 0.0, p)
        return r * r

    ref = np.zeros((toks.size, wl.H))
    for i in range(toks.size):
        for j in range(wl.k):
            e = ids[i, j]
            ref[i] += w[i, j] * (wd[e] @ act(wu[e] @ x[i], wl.I))
        ref[i] *= wl.rsf
        if wl.I_shared:
            su = W.bf16_bits_to_f32(inp["shared_up"]).astype(np.float64)
            sd = W.bf16_bits_to_f32(inp["shared_down"]).astype(np.float64)
            ref[i] += sd @ act(su @ x[i], wl.I_shared)
    nan = np.isnan(ref)
    assert (np.isnan(out) == nan).all()
    if wl.mx_nan:
        assert nan.any()
    assert np.allclose(out[~nan], ref[~nan], rtol=1e-10, atol=1e-12 * np.abs(ref[~nan]).max())
