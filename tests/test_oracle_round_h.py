"""Pins of the oracle's stored-activation option (round_h).

The MoE kernels keep the activation between the two projections as a bf16
tensor, rounded once on the store (vllm.cpp PR #684, the W2 commit: the
relu^2 arm widens to f32, squares and rounds once on the store). With
round_h the oracle applies exactly that rounding (to fp32, then to bf16,
nearest even) to each routed and shared activation and nothing else; by
default it keeps the activation exact. The pins are hand-worked values on a
layer built so that each output element is one activation:
  * (1 + 2^-5)^2 = 1 + 2^-4 + 2^-10 lies below half a bf16 ulp above
    1 + 2^-4: it rounds down;
  * (1 + 2^-4)^2 = 1 + 2^-3 + 2^-8 is exactly half an ulp above 1 + 2^-3:
    the tie goes to the even mantissa, down;
  * (1 + 9/128)^2 = 1 + 2385/16384 lies above 1 + 18/128 + half an ulp: up
    to 1 + 19/128;
and on exact one-hot inputs the option must agree with the fp32 mimic's
expert rows (each a single exact product of a bf16-rounded activation).
"""
import numpy as np

import oracle
from sigmoid_top_routing_amd import workloads as W

U = [1.0 + 2.0 ** -5, 1.0 + 2.0 ** -4, 1.0 + 9.0 / 128.0]
ROUNDED = [1.0 + 2.0 ** -4, 1.0 + 2.0 ** -3, 1.0 + 19.0 / 128.0]


def _hand_layer():
    # two relu^2 experts; the router sends every token to expert 0 with
    # weight sigmoid(0) = 1/2 (no renormalisation); up row n of expert 0 and
    # of the shared expert reads x column 0 with weight U[n]; down row n
    # (routed) and row 8 + n (shared) pick activation n
    H = I = Is = 64
    wl = W.Workload("pin_round_h", T=3, H=H, I=I, E=2, k=1, act="relu2", norm_topk=False,
                    I_shared=Is, rsf=1.0)
    bf = lambda a: W.f32_to_bf16_bits(np.asarray(a, np.float32))
    x = np.zeros((3, H), np.float32)
    x[:, 0] = 1.0
    router_w = np.zeros((2, H), np.float32)
    router_w[1, 0] = -1.0
    w_up = np.zeros((2, I, H), np.float32)
    w_down = np.zeros((2, H, I), np.float32)
    s_up = np.zeros((Is, H), np.float32)
    s_down = np.zeros((H, Is), np.float32)
    for n, u in enumerate(U):
        w_up[0, n, 0] = u
        w_down[0, n, n] = 1.0
        s_up[n, 0] = u
        s_down[8 + n, n] = 1.0
    inp = {"x": bf(x), "router_w": router_w, "bias": np.zeros(2, np.float32),
           "w_up": bf(w_up), "w_down": bf(w_down), "shared_up": bf(s_up),
           "shared_down": bf(s_down)}
    for a in ("x", "w_up", "w_down", "shared_up", "shared_down"):
        assert (W.bf16_bits_to_f32(inp[a]) == {"x": x, "w_up": w_up, "w_down": w_down,
                                                "shared_up": s_up, "shared_down": s_down}[a]).all()
    return wl, inp


def test_round_h_hand_values_routed_and_shared():
    wl, inp = _hand_layer()
    exact, ids, w = oracle.forward_tokens(wl, inp, np.arange(3), want_routing=True)
    stored = oracle.forward_tokens(wl, inp, np.arange(3), round_h=True)
    assert (ids == 0).all() and (w == 0.5).all()
    for n in range(3):
        assert (exact[:, n] == 0.5 * U[n] ** 2).all()           # the definition: exact
        assert (exact[:, 8 + n] == U[n] ** 2).all()
        assert (stored[:, n] == 0.5 * ROUNDED[n]).all()         # routed, rounded
        assert (stored[:, 8 + n] == ROUNDED[n]).all()           # shared, rounded, unscaled
    rest = np.ones(wl.H, bool)
    rest[[0, 1, 2, 8, 9, 10]] = False
    assert (stored[:, rest] == 0).all() and (exact[:, rest] == 0).all()


def test_round_h_matches_the_fp32_mimic_on_one_hot_inputs():
    # relu^2 on one-hot inputs: every projection is one exact product, so
    # the stored activations are the mimic's bf16 epilogue values, and each
    # down row is one exact product of them
    wl = W.Workload("pin_round_h_onehot", T=48, H=128, I=64, E=6, k=3, act="relu2", rsf=2.5,
                    I_shared=64, seed=11)
    inp = W.exact_inputs(wl)
    toks = np.arange(wl.T)
    out, ids, w = oracle.forward_tokens(wl, inp, toks, want_routing=True, round_h=True)
    y, sh, inexact = oracle.expert_rows32(wl, inp, toks, ids)
    assert inexact == 0
    want = wl.rsf * np.einsum("tj,tjh->th", w, y.astype(np.float64)) + sh.astype(np.float64)
    assert np.allclose(out, want, rtol=1e-14, atol=0.0)
    exact = oracle.forward_tokens(wl, inp, toks)
    assert (exact != out).mean() > 0.05                         # the option is visible
