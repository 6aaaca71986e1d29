"""Pins of the oracle's experts and combine.

Closed forms on hand-built layers (one-hot inputs make every projection a
single exact product), the SiLU checked through the identity
silu(g) = g (1 + tanh(g/2)) / 2 rather than the exponential form the oracle
uses, exact rational arithmetic for relu^2, NumPy's float64 matmul on the
textbook single-expert case and on a dense masked form of the whole block,
linearity in the routed scaling factor, and hand-decoded 4-bit rows.

Sources: TileGym PR #187 "Weight layout and routing" (gate_up (E, 2I, H)
with gate rows first, down (E, H, I)); vllm.cpp PR #684 "The seam decision"
and the W2 commit (relu^2 expert h = relu(up x)^2; routed scale on the
finished routed sum, shared term added unscaled); bloomery PR #235 "What"
(relu^2 keeps a non-finite input non-finite); TensorFold PR #1492 "What"
(MLX 4-bit affine experts).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def silu_tanh(g):
    return g * 0.5 * (1.0 + np.tanh(0.5 * g))


# ---------------------------------------------------------------- hand layers

C0, V0 = 5, 1.0      # token 0: one-hot at column 5, value 1
C1, V1 = 40, -2.0    # token 1: one-hot at column 40, value -2; token 2: zeros


def _G(e, n, c):
    return ((n * 5 + e * 3 + c) % 33 - 16) / 8.0


def _U(e, n, c):
    return ((n * 7 + e + 2 * c) % 17 - 8) / 4.0


def _D(e, h):
    return ((h % 5) + 1) / 4.0 * (1.0 if e % 2 == 0 else -1.0)


def _perm(h, e, I):
    return (3 * h + e) % I


def _pack(q):
    """q [..., K] ints in 0..15 -> words [..., K/8], little nibble first."""
    q = np.asarray(q, dtype=np.uint32)
    words = np.zeros(q.shape[:-1] + (q.shape[-1] // 8,), dtype=np.uint32)
    for i in range(8):
        words |= q[..., i::8] << np.uint32(4 * i)
    return words


def hand_layer(act="swiglu", wfmt="bf16", rsf=1.0, I_shared=0):
    H = I = 64
    E, k, T = 4, 2, 3
    wl = W.Workload("hand", T=T, H=H, I=I, E=E, k=k, act=act, wfmt=wfmt, rsf=rsf,
                    I_shared=I_shared)
    x = np.zeros((T, H), np.float32)
    x[0, C0], x[1, C1] = V0, V1
    inp = {"x": W.f32_to_bf16_bits(x),
           "router_w": np.zeros((E, H), np.float32),          # every score is 1/2
           "bias": np.array([0.0, 0.3, 0.2, 0.1], np.float32)}  # picks experts 1, 2
    n_up = wl.n_up
    up = np.zeros((E, n_up, H), np.float32)
    for e in range(E):
        for n in range(I):
            for c in (C0, C1):
                if act == "swiglu":
                    up[e, n, c] = _G(e, n, c)
                    up[e, I + n, c] = _U(e, n, c)
                else:
                    up[e, n, c] = _U(e, n, c)
    down = np.zeros((E, H, I), np.float32)
    for e in range(E):
        for h in range(H):
            down[e, h, _perm(h, e, I)] = _D(e, h)
    if wfmt == "bf16":
        inp["w_up"] = W.f32_to_bf16_bits(up)
        inp["w_down"] = W.f32_to_bf16_bits(down)
    else:
        # affine-4 up rows: q = (n + 2e + c) % 16 at the two live columns
        # (8 elsewhere, where the input is zero), scale 2^-(n % 3) / 4,
        # bias -((e + n) % 4) / 8; the live values are recorded in `up`.
        q = np.full((E, n_up, H), 8, np.int64)
        sc = np.zeros((E, n_up, 1), np.float32)
        bi = np.zeros((E, n_up, 1), np.float32)
        for e in range(E):
            for n in range(n_up):
                sc[e, n, 0] = 2.0 ** -(n % 3) / 4.0
                bi[e, n, 0] = -((e + n) % 4) / 8.0
                for c in (C0, C1):
                    q[e, n, c] = (n + 2 * e + c) % 16
                    up[e, n, c] = sc[e, n, 0] * q[e, n, c] + bi[e, n, 0]
        inp["w_up"] = _pack(q)
        inp["w_up_scales"] = W.f32_to_bf16_bits(sc)
        inp["w_up_biases"] = W.f32_to_bf16_bits(bi)
        # affine-4 down rows are dense: q = (h + i + e) % 16, scale 2^-(h % 3),
        # bias -(e + 1) / 16
        qd = np.zeros((E, H, I), np.int64)
        scd = np.zeros((E, H, 1), np.float32)
        bid = np.zeros((E, H, 1), np.float32)
        for e in range(E):
            for h in range(H):
                qd[e, h] = (h + np.arange(I) + e) % 16
                scd[e, h, 0] = 2.0 ** -(h % 3)
                bid[e, h, 0] = -(e + 1) / 16.0
        inp["w_down"] = _pack(qd)
        inp["w_down_scales"] = W.f32_to_bf16_bits(scd)
        inp["w_down_biases"] = W.f32_to_bf16_bits(bid)
        inp["_down_exact"] = (qd, scd[..., 0], bid[..., 0])
    if I_shared:
        n_sup = 2 * I_shared if act == "swiglu" else I_shared
        su = np.zeros((n_sup, H), np.float32)
        for n in range(n_sup):
            for c in (C0, C1):
                su[n, c] = ((n * 3 + c) % 13 - 6) / 4.0
        sd = np.zeros((H, I_shared), np.float32)
        for h in range(H):
            sd[h, (5 * h) % I_shared] = 0.5
        inp["shared_up"] = W.f32_to_bf16_bits(su)
        inp["shared_down"] = W.f32_to_bf16_bits(sd)
    inp["_up_f"] = up
    return wl, inp


def hand_expected(wl, inp):
    """Closed-form output rows of the hand layer."""
    H, I, k = wl.H, wl.I, wl.k
    w = 0.5 / (1.0 + 1e-6)
    ids = (1, 2)
    out = np.zeros((wl.T, H))
    for t, (c, v) in enumerate(((C0, V0), (C1, V1), (None, 0.0))):
        for e in ids:
            if c is None:
                continue
            upf = inp["_up_f"].astype(np.float64)
            if wl.act == "swiglu":
                g = np.array([v * upf[e, n, c] for n in range(I)])
                u = np.array([v * upf[e, I + n, c] for n in range(I)])
                act = silu_tanh(g) * u
            else:
                u = [Fraction(v) * Fraction(float(upf[e, n, c])) for n in range(I)]
                act = [(ui if ui > 0 else Fraction(0)) ** 2 for ui in u]
            if wl.wfmt == "bf16":
                y = np.array([_D(e, h) * float(act[_perm(h, e, I)]) for h in range(H)])
            else:
                qd, scd, bid = inp["_down_exact"]
                y = np.zeros(H)
                for h in range(H):
                    wrow = [Fraction(float(scd[e, h])) * int(qd[e, h, i]) + Fraction(float(bid[e, h]))
                            for i in range(I)]
                    y[h] = float(sum(wr * (act[i] if isinstance(act[i], Fraction)
                                           else Fraction(float(act[i]))) for i, wr in enumerate(wrow)))
            out[t] += w * y
        out[t] *= wl.rsf
        if wl.I_shared and c is not None:
            Is = wl.I_shared
            su = [((n * 3 + c) % 13 - 6) / 4.0 for n in range(2 * Is)]
            if wl.act == "swiglu":
                g = np.array([v * su[n] for n in range(Is)])
                u = np.array([v * su[Is + n] for n in range(Is)])
                sact = silu_tanh(g) * u
            else:
                u = np.array([v * su[n] for n in range(Is)])
                sact = np.where(u > 0, u, 0.0) ** 2
            out[t] += np.array([0.5 * sact[(5 * h) % Is] for h in range(H)])
    return out


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
@pytest.mark.parametrize("wfmt", ["bf16", "affine4"])
@pytest.mark.parametrize("rsf,I_shared", [(1.0, 0), (2.5, 64)])
def test_hand_layer_closed_form(act, wfmt, rsf, I_shared):
    wl, inp = hand_layer(act, wfmt, rsf, I_shared)
    got, ids, w = oracle.forward_tokens(wl, inp, [0, 1, 2], want_routing=True)
    assert (ids == np.array([[1, 2]] * 3)).all()
    exp = hand_expected(wl, inp)
    assert np.abs(exp).max() > 0.1
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-12 * np.abs(exp).max())
    assert (got[2] == 0).all()


def test_hand_layer_separates_the_readings_it_pins():
    # the closed form must tell apart gate/up order and the place of the
    # routed scale (on the routed sum only, not on the shared term)
    wl, inp = hand_layer("swiglu", "bf16", 2.5, 64)
    exp = hand_expected(wl, inp)
    routed = hand_expected(wl.with_(I_shared=0), inp)
    shared = exp - routed
    scaled_shared = routed + wl.rsf * shared
    assert np.abs(scaled_shared - exp).max() > 1e-3
    swapped = dict(inp)
    I = wl.I
    wu = inp["w_up"]
    swapped["w_up"] = np.ascontiguousarray(np.concatenate([wu[:, I:], wu[:, :I]], axis=1))
    assert np.abs(oracle.forward_tokens(wl, swapped, [0, 1, 2]) - exp).max() > 1e-3


def test_activation_special_values():
    nan, inf = float("nan"), float("inf")
    assert math.isnan(oracle.activate("relu2", 0.0, nan))
    assert oracle.activate("relu2", 0.0, inf) == inf
    assert oracle.activate("relu2", 0.0, -inf) == 0.0
    assert oracle.activate("relu2", 0.0, -2.0) == 0.0
    assert oracle.activate("relu2", 0.0, 3.0) == 9.0
    assert oracle.activate("swiglu", 0.0, 5.0) == 0.0
    assert math.isnan(oracle.activate("swiglu", nan, 1.0))
    for g in (-3.0, -0.5, 0.25, 2.0, 9.0):
        assert math.isclose(oracle.activate("swiglu", g, 1.5), 1.5 * float(silu_tanh(g)),
                            rel_tol=1e-14)


# ---------------------------------------------------------------- affine-4 decode

def test_affine4_decode_hand_cases():
    spec = json.load(open(os.path.join(GOLDEN, "affine4_decode.json")))
    g = spec["group"]
    for case in spec["cases"]:
        K = 128
        codes = np.zeros((1, K // 8), np.uint32)
        if "words_hex" in case:
            for i, hx in enumerate(case["words_hex"]):
                codes[0, i] = int(hx, 16)
        for i, hx in case.get("words_hex_at", {}).items():
            codes[0, int(i)] = int(hx, 16)
        sc = np.array([[int(h, 16) for h in case["scale_bf16_hex"]]], np.uint16)
        bi = np.array([[int(h, 16) for h in case["bias_bf16_hex"]]], np.uint16)
        if sc.shape[1] < K // g:
            sc = np.repeat(sc, K // g, axis=1)
            bi = np.repeat(bi, K // g, axis=1)
        got = oracle.affine4_decode(codes, sc, bi, g)[0]
        if "first16" in case:
            assert list(got[:16]) == case["first16"], case["name"]
        else:
            assert got[case["element"]] == case["value"], case["name"]


# ---------------------------------------------------------------- library cross-checks

def _f64_weights(wl, inp):
    if wl.wfmt == "bf16":
        up = W.bf16_bits_to_f32(inp["w_up"]).astype(np.float64)
        down = W.bf16_bits_to_f32(inp["w_down"]).astype(np.float64)
    else:
        up = np.stack([oracle.affine4_decode(inp["w_up"][e], inp["w_up_scales"][e],
                                             inp["w_up_biases"][e]) for e in range(wl.E)])
        down = np.stack([oracle.affine4_decode(inp["w_down"][e], inp["w_down_scales"][e],
                                               inp["w_down_biases"][e]) for e in range(wl.E)])
    return up, down


def _act(wl, pre, I):
    if wl.act == "swiglu":
        return silu_tanh(pre[..., :I]) * pre[..., I:]
    return np.where(pre > 0, pre, 0.0) ** 2


def _dense(wl, inp):
    """The whole block in dense masked form with NumPy matmuls: every expert
    runs on every token, and a token's mask row keeps only its picks."""
    ids, w = oracle.route(inp["x"], inp["router_w"], inp["bias"], wl.k)
    x = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    up, down = _f64_weights(wl, inp)
    M = np.zeros((wl.T, wl.E))
    for t in range(wl.T):
        for j in range(wl.k):
            M[t, ids[t, j]] += w[t, j]
    out = np.zeros((wl.T, wl.H))
    for e in range(wl.E):
        if not M[:, e].any():
            continue
        y = _act(wl, x @ up[e].T, wl.I) @ down[e].T
        out += M[:, e:e + 1] * y
    out *= wl.rsf
    if wl.I_shared:
        su = W.bf16_bits_to_f32(inp["shared_up"]).astype(np.float64)
        sd = W.bf16_bits_to_f32(inp["shared_down"]).astype(np.float64)
        out += _act(wl, x @ su.T, wl.I_shared) @ sd.T
    return out


@pytest.mark.parametrize("name", ["mid_swiglu", "mid_relu2_shared", "mid_affine4",
                                  "mid_affine4_relu2", "tiny_t64_e8_k2"])
def test_dense_masked_equivalence(name):
    wl = W.by_name(name)
    if wl.T > 300:
        wl = wl.with_(T=300)
    inp = W.generate(wl)
    got = oracle.forward_tokens(wl, inp, np.arange(wl.T))
    ref = _dense(wl, inp)
    assert (np.isnan(got) == np.isnan(ref)).all()
    fin = ~np.isnan(ref)
    rms = np.sqrt(np.mean(ref[fin] ** 2))
    assert np.abs(got[fin] - ref[fin]).max() <= 1e-10 * rms


def test_single_expert_textbook_mlp():
    # E = 1, k = 1: out = rsf * s/(s + 1e-6) * W_d act(W_up x) + shared
    wl = W.Workload("one", T=7, H=128, I=192, E=1, k=1, rsf=1.75, I_shared=64, seed=9)
    for act in ("swiglu", "relu2"):
        wl = wl.with_(act=act)
        inp = W.generate(wl)
        got, ids, w = oracle.forward_tokens(wl, inp, np.arange(wl.T), want_routing=True)
        _, _, _, s = oracle.route(inp["x"], inp["router_w"], inp["bias"], 1, want_scores=True)
        s = s[:, 0].astype(np.float64)
        assert np.allclose(w[:, 0], s / (s + 1e-6), rtol=1e-15)
        x = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
        up = W.bf16_bits_to_f32(inp["w_up"][0]).astype(np.float64)
        dn = W.bf16_bits_to_f32(inp["w_down"][0]).astype(np.float64)
        su = W.bf16_bits_to_f32(inp["shared_up"]).astype(np.float64)
        sd = W.bf16_bits_to_f32(inp["shared_down"]).astype(np.float64)
        routed = _act(wl, x @ up.T, wl.I) @ dn.T
        shared = _act(wl, x @ su.T, wl.I_shared) @ sd.T
        ref = wl.rsf * (s / (s + 1e-6))[:, None] * routed + shared
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_routed_scale_is_linear_and_spares_the_shared_term():
    wl = W.MID["mid_relu2_shared"].with_(T=40)
    inp = W.generate(wl)
    toks = np.arange(wl.T)
    o0 = oracle.forward_tokens(wl.with_(rsf=0.0), inp, toks)   # shared expert alone
    o1 = oracle.forward_tokens(wl.with_(rsf=1.0), inp, toks)
    o25 = oracle.forward_tokens(wl.with_(rsf=2.5), inp, toks)
    assert np.allclose(o25 - o0, 2.5 * (o1 - o0), rtol=1e-12, atol=1e-12 * np.abs(o1).max())
    assert np.abs(o0).max() > 0 and np.abs(o1 - o0).max() > 0


def test_nan_rows_stay_in_their_rows():
    wl = W.TINY
    inp = W.generate(wl)
    out = oracle.forward_tokens(wl, inp, np.arange(wl.T))
    bad = np.isnan(out).any(axis=1)
    assert set(np.nonzero(bad)[0]) == set(wl.nan_rows)
    assert np.isnan(out[list(wl.nan_rows)]).all()
    assert np.isfinite(out[~bad]).all()
    assert (out[wl.zero_tie_row] == 0).all()


# ---------------------------------------------------------------- swiglu_limit
# GLM's experts clamp the SwiGLU inputs at swiglu_limit (TensorFold issue
# #548, the GLM experts' untested paths: at limit 10 about 16 % of gate and
# 33 % of up pre-activations clamp, one side for the gate, both for up).

def silu_exp(g):
    return g / (1.0 + math.exp(-g))


def test_swiglu_limit_special_values():
    nan, inf = float("nan"), float("inf")
    L = 10.0
    cases = [  # (g, u, expected)
        (20.0, 3.0, silu_exp(10.0) * 3.0),      # gate capped above
        (-20.0, 3.0, silu_exp(-20.0) * 3.0),    # never below
        (2.0, 15.0, silu_exp(2.0) * 10.0),      # up capped above
        (2.0, -15.0, silu_exp(2.0) * -10.0),    # and below
        (9.5, -9.5, silu_exp(9.5) * -9.5),      # inside: untouched
        (inf, 1.0, silu_exp(10.0)),
        (1.0, -inf, silu_exp(1.0) * -10.0),
    ]
    for g, u, want in cases:
        assert math.isclose(oracle.activate("swiglu", g, u, L), want, rel_tol=1e-14), (g, u)
    assert math.isnan(oracle.activate("swiglu", nan, 1.0, L))
    assert math.isnan(oracle.activate("swiglu", 1.0, nan, L))
    # limit 0 is no clamp
    assert math.isclose(oracle.activate("swiglu", 20.0, 15.0, 0.0), silu_exp(20.0) * 15.0,
                        rel_tol=1e-14)
    # relu^2 takes no limit
    assert oracle.activate("relu2", 0.0, 30.0, L) == 900.0


def test_swiglu_limit_changes_exactly_the_clamped_tokens():
    # Tokens none of whose routed or shared pre-activations pass the limit
    # keep the limit-0 output bit for bit; every other token changes.
    wl = W.MID["mid_swiglu_limit"].with_(T=40, x_std=6.5)
    inp = W.generate(wl)
    toks = np.arange(wl.T)
    out_l, ids, _ = oracle.forward_tokens(wl, inp, toks, want_routing=True)
    out_0 = oracle.forward_tokens(wl.with_(swiglu_limit=0.0), inp, toks)
    x = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wu = W.bf16_bits_to_f32(inp["w_up"]).astype(np.float64)
    su = W.bf16_bits_to_f32(inp["shared_up"]).astype(np.float64)
    L, I, Is = wl.swiglu_limit, wl.I, wl.I_shared
    changed = 0
    for t in range(wl.T):
        pre = [wu[e] @ x[t] for e in ids[t]] + [su @ x[t]]
        n = [I] * wl.k + [Is]
        hit = any((p[:m] > L).any() or (np.abs(p[m:]) > L).any() for p, m in zip(pre, n))
        same = (out_l[t] == out_0[t]).all()
        assert same != hit, t
        changed += hit
    assert 0 < changed < wl.T


def test_swiglu_limit_workload_clamps_the_stated_fractions():
    # the input recipe of the limit case: gate one-sided ~16 %, up two-sided ~33 %
    wl = W.MID["mid_swiglu_limit"]
    inp = W.generate(wl)
    x = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wu = W.bf16_bits_to_f32(inp["w_up"][:4]).astype(np.float64)
    g = np.einsum("th,enh->ten", x, wu[:, :wl.I])
    u = np.einsum("th,enh->ten", x, wu[:, wl.I:])
    L = wl.swiglu_limit
    assert 0.13 < (g > L).mean() < 0.19
    assert 0.28 < (np.abs(u) > L).mean() < 0.38
