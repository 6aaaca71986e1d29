"""The seeded input generator: determinism, storage formats, constructed rows."""
import hashlib

import numpy as np
import pytest

from sigmoid_top_routing_amd import workloads as W


def _digest(inp):
    h = hashlib.sha256()
    for k in sorted(inp):
        h.update(k.encode())
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", sorted(W.MID) + ["tiny_t64_e8_k2"])
def test_generation_is_deterministic(name):
    wl = W.by_name(name)
    assert _digest(W.generate(wl)) == _digest(W.generate(wl))


def test_shapes_and_dtypes():
    for wl in [W.TINY, *W.MID.values()]:
        inp = W.generate(wl)
        assert inp["x"].shape == (wl.T, wl.H) and inp["x"].dtype == np.uint16
        assert inp["router_w"].shape == (wl.E, wl.H) and inp["router_w"].dtype == np.float32
        assert inp["bias"].shape == (wl.E,)
        if wl.wfmt == "bf16":
            assert inp["w_up"].shape == (wl.E, wl.n_up, wl.H)
            assert inp["w_down"].shape == (wl.E, wl.H, wl.I)
        elif wl.wfmt == "fp8":
            assert inp["w_up"].shape == (wl.E, wl.n_up, wl.H) and inp["w_up"].dtype == np.uint8
            assert inp["w_up_scales"].shape == (wl.E, wl.n_up // 128, wl.H // 128)
            assert inp["w_down_scales"].dtype == np.float32
            assert inp["w_down_scales"].shape == (wl.E, wl.H // 128, wl.I // 128)
            assert not ((inp["w_up"] & 0x7F) == 0x7F).any()      # no NaN codes
        elif wl.wfmt == "mxfp4":
            assert inp["w_up"].shape == (wl.E, wl.n_up, wl.H // 2) and inp["w_up"].dtype == np.uint8
            assert inp["w_up_scales"].shape == (wl.E, wl.n_up, wl.H // 32)
            assert inp["w_down_scales"].shape == (wl.E, wl.H, wl.I // 32)
            assert (inp["w_up_scales"] != 255).all()              # NaN only where planted
        elif wl.wfmt == "nvfp4":
            assert inp["w_up"].shape == (wl.E, wl.n_up, wl.H // 2) and inp["w_up"].dtype == np.uint8
            assert inp["w_down"].shape == (wl.E, wl.H, wl.I // 2)
            assert inp["w_up_scales"].shape == (wl.E, wl.n_up, wl.H // 16)
            assert inp["w_down_scales"].shape == (wl.E, wl.H, wl.I // 16)
            assert inp["w_up_scales"].dtype == np.uint8
            assert not (inp["w_up_scales"] & 0x80).any()          # positive scales
            assert not ((inp["w_up_scales"] & 0x7F) == 0x7F).any()  # never NaN
            assert inp["w_up_global"].shape == (wl.E,) and inp["w_up_global"].dtype == np.float32
        else:
            assert inp["w_up"].shape == (wl.E, wl.n_up, wl.H // 8)
            assert inp["w_up"].dtype == np.uint32
            assert inp["w_up_scales"].shape == (wl.E, wl.n_up, wl.H // 64)
            assert inp["w_down"].shape == (wl.E, wl.H, wl.I // 8)
            assert inp["w_down_biases"].shape == (wl.E, wl.H, wl.I // 64)
        if wl.I_shared:
            assert inp["shared_down"].shape == (wl.H, wl.I_shared)


def test_bf16_rounding_is_nearest_even():
    one = 1.0
    half_ulp = 2.0 ** -8          # bf16 spacing at 1 is 2^-7
    vals = np.array([one + half_ulp, one + 3 * half_ulp, one + half_ulp * 1.01, -one - half_ulp,
                     np.nan, np.inf, -0.0], np.float32)
    b = W.f32_to_bf16_bits(vals)
    back = W.bf16_bits_to_f32(b)
    assert back[0] == 1.0                      # tie -> even (1.0)
    assert back[1] == 1.0 + 2 * 2.0 ** -7      # tie -> even (1 + 2^-6)
    assert back[2] == 1.0 + 2.0 ** -7          # above the tie -> up
    assert back[3] == -1.0
    assert b[4] == 0x7FC0 and back[5] == np.inf and b[6] == 0x8000


def test_distributions_roughly_as_stated():
    wl = W.MID["mid_swiglu"]
    inp = W.generate(wl)
    x = W.bf16_bits_to_f32(inp["x"])
    w = W.bf16_bits_to_f32(inp["w_up"])
    assert abs(x.std() - 1.0) < 0.02 and abs(w.std() - 0.02) < 0.001
    assert abs(inp["router_w"].std() - 0.02) < 0.002
    assert inp["bias"].min() >= -0.05 and inp["bias"].max() <= 0.05
    a = W.MID["mid_affine4"]
    ia = W.generate(a)
    sc = W.bf16_bits_to_f32(ia["w_up_scales"])
    assert sc.min() >= 0.0049 and sc.max() <= 0.0201
    nib = (ia["w_up"][..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    counts = np.bincount(nib.reshape(-1), minlength=16)
    assert counts.min() > 0.9 * counts.mean()


def test_constructed_rows():
    wl = W.TINY
    inp = W.generate(wl)
    for r in wl.nan_rows:
        assert (inp["x"][r] == 0x7FC0).all()
    assert (inp["x"][wl.zero_tie_row] == 0).all()
    assert (inp["bias"][[1, 4, 6]] == np.float32(0.125)).all()
    assert np.delete(inp["bias"], [1, 4, 6]).max() < 0.125
    row = inp["x"][wl.onehot_tie_row]
    assert row[wl.tie_col] == 0x3F80 and np.count_nonzero(row) == 1
    assert inp["router_w"][2, wl.tie_col] == 2.0 and inp["router_w"][5, wl.tie_col] == 2.0
    assert inp["bias"][5] == inp["bias"][2]


def test_decode_shares_prefill_weights():
    a = W.PREFILL.with_(T=4)
    b = W.DECODE.with_(T=4)
    ia, ib = W.generate(a.with_(H=128, I=64)), W.generate(b.with_(H=128, I=64))
    assert (ia["w_up"] == ib["w_up"]).all() and (ia["router_w"] == ib["router_w"]).all()
    assert not (ia["x"] == ib["x"]).all()


def test_affine4_boost():
    wl = W.AFFINE4.with_(H=128, I=64)
    inp = W.generate(wl, need_x=False)
    b = inp["bias"]
    assert all(1.94 < b[e] < 2.06 for e in wl.boosted)
    assert np.abs(np.delete(b, list(wl.boosted))).max() <= 0.05
