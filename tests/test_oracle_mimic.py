"""Pins of the oracle's fp32 mimic of the engine's own order.

The mimic (oracle_combine32, oracle_epilogue32, oracle_expert_rows32) is
what the GPU's fp32 output is compared with bit for bit, on data where every
expert projection is a single exact product. Its pins here are values worked
out by hand or by exact rational arithmetic, never the mimic's own formula:

* the combine: an fma chain over j ascending (a 2^24 cancellation whose
  result depends on the order, and a product whose fused and unfused sums
  differ), the routed scale applied once to the finished sum and the shared
  term added after it, unscaled (vllm.cpp PR #684, the W2 and review-repairs
  commits), and the folded form telling the two apart on decimal-grid data;
* the epilogue: relu^2 of -inf, +inf, NaN and -0, a one-ulp and a tie case
  of the rounding to bf16 (to nearest, ties to even), and the saturated
  SwiGLU (gate above 17: the fp32 sigmoid is 1, silu(g) u is g u);
* the expert rows on one-hot inputs: every value is the indexed product the
  construction promises, and nothing is inexact.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W

F32 = np.float32


def f32(*v):
    return np.array(v, dtype=F32)


def combine(w, y, shared=None, rsf=1.0, fold=False):
    w = np.asarray(w, F32).reshape(1, -1)
    y = np.asarray(y, F32).reshape(1, w.shape[1], -1)
    sh = None if shared is None else np.asarray(shared, F32).reshape(1, -1)
    return oracle.combine32(w, y, sh, rsf, fold)[0]


def test_combine_is_an_fma_chain_over_j_ascending():
    # 2^24 + 1 rounds back to 2^24 (a tie, to even): ascending j gives
    # ((0 + 2^24) + 1) - 2^24 = 0; descending j would give 1
    b = 2.0 ** 24
    assert combine([1, 1, 1], [[b], [1], [-b]])[0] == 0.0
    assert combine([1, 1, 1], [[-b], [1], [b]])[0] == 1.0
    # fused: -1 + (1 + 2^-12)^2 = 2^-11 + 2^-24 exactly; an unfused product
    # would round (1 + 2^-12)^2 to 1 + 2^-11 first and give 2^-11
    a = 1.0 + 2.0 ** -12
    assert combine([1, a], [[-1], [a]])[0] == F32(2.0 ** -11 + 2.0 ** -24)
    # k = 1: the correctly rounded product (exact rational, then the one
    # rounding of a value that fits a double)
    rng = np.random.default_rng(0)
    w = rng.uniform(0.5, 2, 64).astype(F32)
    y = rng.uniform(-4, 4, 64).astype(F32)
    got = np.array([combine([wi], [[yi]])[0] for wi, yi in zip(w, y)])
    exact = np.array([F32(float(Fraction(float(wi)) * Fraction(float(yi)))) for wi, yi in zip(w, y)])
    assert (got.view(np.uint32) == exact.view(np.uint32)).all()


def test_routed_scale_once_after_the_sum_and_shared_unscaled():
    # rsf 2, one expert, shared 1: (1 * 1) * 2 + 1 = 3 (scaling the shared
    # term or adding it before the scale gives 4)
    assert combine([1], [[1]], shared=[1], rsf=2.0)[0] == 3.0
    # rsf applied after the sum: w = (1, 1), y = (1, 2^-24), rsf 3. The sum
    # 1 + 2^-24 is half an ulp above 1 and rounds to 1 (ties to even), so the
    # engine gives 3 * 1 = 3. Folded, fma(3, 2^-24, 3) = 3 + 0.75 ulp(3)
    # rounds up to 3 + 2^-22.
    assert combine([1, 1], [[1], [2.0 ** -24]], rsf=3.0)[0] == F32(3.0)
    assert combine([1, 1], [[1], [2.0 ** -24]], rsf=3.0, fold=True)[0] == F32(3.0 + 2.0 ** -22)
    # at rsf 1 the two forms are the same function
    rng = np.random.default_rng(1)
    w = rng.uniform(0, 0.5, (4,)).astype(F32)
    y = rng.standard_normal((4, 32)).astype(F32)
    a = combine(w, y, rsf=1.0)
    b = combine(w, y, rsf=1.0, fold=True)
    assert (a.view(np.uint32) == b.view(np.uint32)).all()


def test_folded_form_differs_on_decimal_grid_data():
    # decimal weights and rsf 0.7 (neither exact in binary): the folded form
    # rounds rsf * w_j once per term, the engine's form once at the end
    w = f32(0.1, 0.2, 0.3, 0.4)
    y = (np.arange(4 * 256, dtype=np.float64).reshape(4, 256) % 97 / 10.0 - 4.8).astype(F32)
    a = combine(w, y, rsf=0.7)
    b = combine(w, y, rsf=0.7, fold=True)
    assert (a.view(np.uint32) != b.view(np.uint32)).mean() > 0.2


def test_epilogue_relu2_special_values_and_rounding():
    ep = lambda u: int(oracle.epilogue32("relu2", 0.0, [u])[0])
    assert ep(float("-inf")) == 0x0000            # (u < 0 ? 0 : u)^2
    assert ep(float("inf")) == 0x7F80             # +inf passes
    assert ep(float("nan")) & 0x7FFF > 0x7F80     # NaN passes
    assert ep(-0.0) == 0x0000                     # (-0)^2 = +0
    assert ep(-3.0) == 0x0000
    assert ep(3.0) == 0x4110                      # 9
    # (1 + 2^-7)^2 = 1 + 2^-6 + 2^-14: below half an ulp (2^-8) -> 1 + 2^-6
    assert ep(1.0 + 2.0 ** -7) == 0x3F82
    # (1 + 2^-4 + 2^-7)^2 = 1 + 2^-3 + 2^-6 + 2^-8 + 2^-11 + 2^-14: above the
    # half ulp -> rounds up to 1 + 2^-3 + 2^-6 + 2^-7
    assert ep(1.0 + 2.0 ** -4 + 2.0 ** -7) == 0x3F83 + 0x10


def _rne_bf16(q: Fraction) -> int:
    """bf16 bits of a positive normal rational, round to nearest, ties to even
    (by hand: scale to 8 significant bits, compare the remainder to one half)."""
    e = 0
    while q >= 2:
        q /= 2
        e += 1
    while q < 1:
        q *= 2
        e -= 1
    m = q * 128                                    # 1.xxxxxxx -> 128..255.99
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 256:
        lo, e = 128, e + 1
    return ((e + 127) << 7) | (lo - 128)


def test_epilogue_rounding_ties_to_even_by_exact_arithmetic():
    # every bf16 u in [1, 2): u^2 exact as a rational, rounded by hand; ties
    # (a remainder of exactly one half) occur and must go to even
    ties = 0
    for mant in range(128):
        u = 1.0 + mant / 128.0
        q = Fraction(u) * Fraction(u)
        m = q / (2 if q >= 2 else 1) * 128
        ties += (m - m.numerator // m.denominator) == Fraction(1, 2)
        assert int(oracle.epilogue32("relu2", 0.0, [u])[0]) == _rne_bf16(q), u
    assert ties > 0


def test_epilogue_saturated_swiglu_is_the_product():
    ep = lambda g, u: int(oracle.epilogue32("swiglu", g, [u])[0])
    assert ep(32.0, 3.0) == 0x42C0                 # 96
    assert ep(24.5, -1.25) == 0xC1F5               # -30.625, exact in bf16
    # 127 (1 + 2^-7) = 127.9921875 rounds up to 128
    assert ep(127.0, 1.0 + 2.0 ** -7) == 0x4300
    for g in (24.0, 40.5, 63.0):
        for u in (0.375, -2.25, 3.96875):
            assert ep(g, u) == _rne_bf16(Fraction(g) * Fraction(abs(u))) | (0x8000 if u < 0 else 0)


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_expert_rows_on_one_hot_inputs_are_the_indexed_products(act):
    wl = W.Workload("mimic_" + act, T=40, H=128, I=64, E=6, k=3, act=act, rsf=2.5,
                    I_shared=128, seed=7)
    inp = W.exact_inputs(wl)
    ids = np.stack([np.arange(40) % 6, (np.arange(40) + 1) % 6, (np.arange(40) + 3) % 6],
                   axis=1).astype(np.int32)
    toks = np.arange(40)
    y, sh, inexact = oracle.expert_rows32(wl, inp, toks, ids)
    assert inexact == 0
    val = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    n = np.arange(wl.H)
    for t in (0, 7, 39):
        c = int(W.onehot_col(t, wl.H))
        for j in range(wl.k):
            e = int(ids[t, j])
            col = (7 * n + 3 * e) % wl.I
            if act == "relu2":
                hv = oracle.epilogue32("relu2", 0.0, val(inp["w_up"][e, :, c]))
            else:
                hv = oracle.epilogue32("swiglu", val(inp["w_up"][e, :wl.I, c]),
                                       val(inp["w_up"][e, wl.I:, c]))
            expect = val(inp["w_down"][e, n, col]) * val(hv[col])
            assert (y[t, j].astype(np.float64) == expect).all()
        col = (7 * n + 3 * wl.E) % wl.I_shared
        Is = wl.I_shared
        if act == "relu2":
            hs = oracle.epilogue32("relu2", 0.0, val(inp["shared_up"][:, c]))
        else:
            hs = oracle.epilogue32("swiglu", val(inp["shared_up"][:Is, c]),
                                   val(inp["shared_up"][Is:, c]))
        assert (sh[t].astype(np.float64) == val(inp["shared_down"][n, col]) * val(hs[col])).all()


def test_expert_rows_count_inexact_projections():
    # dense random weights: the fp32 projections are rounded, and counted
    wl = W.Workload("mimic_dense", T=4, H=128, I=64, E=2, k=1, act="relu2", seed=8)
    inp = W.generate(wl)
    _, _, inexact = oracle.expert_rows32(wl, inp, np.arange(4), np.zeros((4, 1), np.int32))
    assert inexact > 100
