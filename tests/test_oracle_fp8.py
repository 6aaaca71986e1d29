"""Pins of the oracle's block-FP8 experts (TensorFold issue #548: the
block-FP8 linears and experts of the CUDA branches, 128 x 128 scales).

The OCP E4M3 decode is checked against hand-computed codes and the format's
structure (254 finite values, monotone in the code, sign symmetric); the
block scales against a dense float64 evaluation of the whole layer whose
scales are laid out with NumPy's repeat, not the oracle's index arithmetic.
"""
import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W


def test_e4m3_hand_values():
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0xB8: -1.0, 0x7E: 448.0,
             0x77: 240.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6,
             0x30: 0.5, 0x29: 1.125 * 2.0 ** -2, 0xFE: -448.0}
    codes = np.array(sorted(table), np.uint8)
    got = oracle.fp8_decode(codes)
    assert list(got) == [table[c] for c in sorted(table)]
    z = oracle.fp8_decode([0x80])[0]
    assert z == 0.0 and np.signbit(z)
    assert np.isnan(oracle.fp8_decode([0x7F, 0xFF])).all()


def test_e4m3_structure():
    v = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    pos, neg = v[1:127], v[129:255]
    assert np.isfinite(v).sum() == 254
    assert (np.diff(pos) > 0).all() and pos[-1] == 448.0
    assert (neg == -pos).all()
    # within a binade the 8 codes are evenly spaced; subnormals continue the
    # spacing of the first binade
    assert np.allclose(np.diff(v[0:16]), 2.0 ** -9)


@pytest.mark.parametrize("name", ["mid_fp8", "mid_fp8_relu2", "mid_fp8_wide"])
def test_fp8_layer_matches_dense_float64(name):
    # mid_fp8_relu2 holds e4m3 NaN codes in three down rows: the tokens
    # routed to those experts get NaN in exactly those output columns
    wl = W.by_name(name)
    inp = W.generate(wl)
    toks = np.arange(12)
    out, ids, w = oracle.forward_tokens(wl, inp, toks, want_routing=True)

    def dense(codes, scales):
        E, N, K = codes.shape
        s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=1), 128, axis=2)
        return oracle.fp8_decode(codes.reshape(-1)).reshape(E, N, K) * s

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
    if wl.fp8_nan:
        hit = {(e, h) for e, h in wl.fp8_nan}
        expect = np.zeros_like(nan)
        for i in range(toks.size):
            for e, h in hit:
                if e in ids[i]:
                    expect[i, h] = True
        assert expect.any() and (nan == expect).all()
    assert np.allclose(out[~nan], ref[~nan], rtol=1e-10, atol=1e-12 * np.abs(ref[~nan]).max())
