"""Parity of the fused residual add + RMSNorm (moe_add_rmsnorm) with the
oracle (TensorFold issue #548: RMSNorm and the fused add + RMSNorm among the
shared layer pieces, a row's bits the same at every row count).

Bars: the residual stream is bf16 of an fp32 sum on both sides, so it is
bit-exact (NaN positions compared as NaN). x is bf16 of a float64 value on
the oracle's side and of an fp32 computation here: every element lies within
one bf16 ulp of the exact value, and all but a few rounding ties (at most
1 in 1000) are its bf16 rounding exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev16(a):
    return torch.from_numpy(a.view(np.int16)).to(DEV)


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def poisoned(shape):
    t = torch.empty(shape, dtype=torch.int16, device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t


def check(res_gpu, x_gpu, res_ref, x_ref):
    nan = np.isnan(W.bf16_bits_to_f32(res_ref))
    assert (np.isnan(W.bf16_bits_to_f32(res_gpu)) == nan).all()
    assert (res_gpu[~nan] == res_ref[~nan]).all()
    xg = W.bf16_bits_to_f32(x_gpu).astype(np.float64)
    xnan = np.isnan(x_ref)
    assert (np.isnan(xg) == xnan).all()
    ref = x_ref[~xnan]
    got = xg[~xnan]
    rounded = W.f32_to_bf16_bits(ref.astype(np.float32))
    ulp = np.spacing(np.abs(W.bf16_bits_to_f32(rounded))) * 2.0 ** 16   # bf16 spacing
    assert (np.abs(got - ref) <= ulp + 1e-38).all()
    exact = (W.f32_to_bf16_bits(got.astype(np.float32)) == rounded).mean() if got.size else 1.0
    assert exact >= 0.999, exact


def run(d, T, H, in_place=False):
    res = dev16(d["residual"])
    h = dev16(d["h"]) if d["h"] is not None else None
    g = dev16(d["gamma"])
    x = poisoned((T, H))
    res_out = res if in_place else poisoned((T, H))
    lib.add_rmsnorm(res, g, d["eps"], h=h, residual_out=res_out, x=x)
    torch.cuda.synchronize()
    return host16(res_out), host16(x)


@pytest.mark.parametrize("with_h", [True, False])
@pytest.mark.parametrize("T,H", [(1, 64), (3, 2048), (4096, 2048), (100, 2688), (7, 8192),
                                 (33, 576), (2, 7680)])
def test_add_rmsnorm_matches_oracle(T, H, with_h):
    d = W.norm_inputs(T, H, seed=T * 31 + H, with_h=with_h)
    d["residual"][0, :] = 0                              # a zero row: x = 0
    if T > 2:
        d["residual"][2, 5] = W.BF16_NAN                 # NaN stays in its row
    res_gpu, x_gpu = run(d, T, H)
    res_ref, x_ref = oracle.add_rmsnorm(d["h"], d["residual"], d["gamma"], d["eps"])
    check(res_gpu, x_gpu, res_ref, x_ref)
    if not with_h:
        assert (x_gpu[0] == 0).all()


def test_add_rmsnorm_in_place_residual():
    T, H = 64, 2048
    d = W.norm_inputs(T, H, seed=5)
    res_ref, x_ref = oracle.add_rmsnorm(d["h"], d["residual"], d["gamma"], d["eps"])
    res_gpu, x_gpu = run(d, T, H, in_place=True)
    check(res_gpu, x_gpu, res_ref, x_ref)


def test_add_rmsnorm_rows_do_not_depend_on_the_row_count():
    T, H = 4096, 2048
    d = W.norm_inputs(T, H, seed=9)
    res_all, x_all = run(d, T, H)
    for t in (0, 1, 2047, 4095):
        one = {"h": d["h"][t:t + 1].copy(), "residual": d["residual"][t:t + 1].copy(),
               "gamma": d["gamma"], "eps": d["eps"]}
        res1, x1 = run(one, 1, H)
        assert (res1[0] == res_all[t]).all() and (x1[0] == x_all[t]).all(), t
