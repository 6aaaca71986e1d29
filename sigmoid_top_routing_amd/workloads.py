"""Seeded synthetic workloads for the sigmoid top-k routed MoE block.

This module only draws numbers. It holds no step of the block's arithmetic:
no router, no sigmoid, no top-k, no expert MLP. Both the HIP path and the
CPU oracle are fed from here, and nothing here depends on either of them.

Shapes follow the MoE blocks the pages rebuild:
  * LFM2-8B-A1B: 32 experts, top-4, SwiGLU experts with a fused gate_up
    weight (E, 2I, H), gate rows first, and down (E, H, I)
    (TileGym PR #187, "Weight layout and routing").
  * Nemotron-H: non-gated relu^2 experts (up (E, I, H), down (E, H, I)), a
    routed scaling factor on the routed sum and an unscaled shared expert
    (vllm.cpp PR #684, "The seam decision" and the W2 commit message).
  * MLX 4-bit affine experts, group 64 (TensorFold PR #1492, "What").

Every tensor is drawn in fp32 from NumPy's PCG64 and, where the layer stores
bf16, rounded to bf16 by round-to-nearest-even. The draws come in a fixed
order from ``np.random.SeedSequence([0x5EED, seed]).spawn(10)``:
x, router weight, expert bias, up weight, down weight, shared up, shared
down, 4-bit codes, 4-bit scales, 4-bit biases. Long draws are taken in
chunks of 2**24 values from one generator, so the stream is fixed.

Affine-4 packing (our convention, the inputs being synthetic): element c of
a row lives in 32-bit word c // 8 at bits 4 * (c % 8) (little nibble
first); the scale and bias of element c are entry c // 64 of the row.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 24
BF16_NAN = 0x7FC0
BF16_ONE = 0x3F80


@dataclass(frozen=True)
class Workload:
    """One synthetic MoE-block workload.

    act: "swiglu" (gate_up (E, 2I, H), gate rows first) or "relu2"
    (up (E, I, H)). wfmt: "bf16" or "affine4" (group 64). score: "sigmoid"
    or "softmax" router scores. swiglu_limit: 0, or the cap L > 0 of the
    SwiGLU inputs (gate <= L, |up| <= L).
    """
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    act: str = "swiglu"
    wfmt: str = "bf16"
    rsf: float = 1.0
    I_shared: int = 0
    norm_topk: bool = True
    norm_eps: float = 1e-6
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    bias_lo: float = -0.05
    bias_hi: float = 0.05
    seed: int = 0
    weight_seed: int | None = None   # draw weights from another seed's stream
    boost: float = 0.0
    boosted: tuple = ()
    nan_rows: tuple = ()
    zero_tie_row: int | None = None  # x row of zeros + triple bias tie
    onehot_tie_row: int | None = None  # one-hot x row + two equal logits
    zero_rows: tuple = ()             # x rows of zeros, bias untouched
    posinf_rows: tuple = ()           # x rows with +inf at column tie_col
    neginf_rows: tuple = ()           # x rows with -inf at column tie_col
    tie_col: int = 7
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    fp8_exp_mu: float = 13.0          # block-FP8 codes: exponent field round(N(mu, sd))
    fp8_exp_sd: float = 1.0
    fp8_nan: tuple = ()               # (expert, row) of w_down rows holding one e4m3 NaN
    global_lo: float = 3e-5           # NVFP4: global scale of each expert matrix, U(lo, hi)
    global_hi: float = 8e-5
    mx_exp_mu: float = 120.0          # MXFP4: E8M0 scale byte round(N(mu, sd))
    mx_exp_sd: float = 1.0
    mx_nan: tuple = ()                # (expert, row) of w_down rows with one NaN scale (0xFF)
    qbias_lo: float = -0.1
    qbias_hi: float = 0.1
    group: int = 64
    score: str = "sigmoid"
    swiglu_limit: float = 0.0

    @property
    def A(self) -> int:
        return self.T * self.k

    @property
    def n_up(self) -> int:
        return 2 * self.I if self.act == "swiglu" else self.I

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of this block, in order: a tiny case the oracle runs
# whole, the LFM2-MoE-shaped prefill chunk, the decode step on the same
# weights, the Nemotron-H-shaped relu^2 block with a shared expert, and the
# 4-bit affine experts with four boosted experts.
TINY = Workload("tiny_t64_e8_k2", T=64, H=128, I=256, E=8, k=2, bias_lo=-0.1, bias_hi=0.1,
                seed=0, nan_rows=(5, 17), zero_tie_row=30, onehot_tie_row=47)
PREFILL = Workload("lfm2_prefill_t4096", T=4096, H=2048, I=1792, E=32, k=4, seed=1)
DECODE = Workload("lfm2_decode_t8", T=8, H=2048, I=1792, E=32, k=4, seed=2, weight_seed=1)
RELU2 = Workload("nemotron_relu2_t2048", T=2048, H=2688, I=1856, E=128, k=6, act="relu2",
                 rsf=2.5, I_shared=3712, bias_lo=-0.1, bias_hi=0.1, seed=3)
AFFINE4 = Workload("affine4_t1024", T=1024, H=2048, I=1792, E=32, k=4, wfmt="affine4", seed=4,
                   boost=2.0, boosted=(3, 11, 19, 27))

CONFIGS = [TINY, PREFILL, DECODE, RELU2, AFFINE4]

# Mid-sized workloads for parity: small enough that the oracle computes every
# token in seconds, large enough to span several tiles with ragged tails.
MID = {
    "mid_swiglu": Workload("mid_swiglu", T=600, H=512, I=320, E=16, k=4, seed=100),
    "mid_swiglu_bigseg": Workload("mid_swiglu_bigseg", T=1100, H=256, I=384, E=4, k=2, seed=101),
    "mid_relu2_shared": Workload("mid_relu2_shared", T=300, H=384, I=192, E=24, k=6, act="relu2",
                                 rsf=2.5, I_shared=448, bias_lo=-0.1, bias_hi=0.1, seed=102),
    "mid_affine4": Workload("mid_affine4", T=256, H=512, I=256, E=8, k=2, wfmt="affine4",
                            seed=103),
    "mid_affine4_relu2": Workload("mid_affine4_relu2", T=200, H=256, I=320, E=12, k=3,
                                  act="relu2", wfmt="affine4", rsf=1.5, I_shared=192, seed=104),
    "mid_nan_ties": Workload("mid_nan_ties", T=333, H=320, I=192, E=16, k=8, bias_lo=-0.1,
                             bias_hi=0.1, seed=105, nan_rows=(0, 100, 332), zero_tie_row=7,
                             onehot_tie_row=200, tie_col=3),
    "mid_e256_k8": Workload("mid_e256_k8", T=96, H=192, I=128, E=256, k=8, seed=106),
    # 4-bit experts whose down projection has K = I = 64 (the staged kernel
    # with the decode in its loads, at prompt and decode sizes)
    "mid_affine4_i64": Workload("mid_affine4_i64", T=200, H=256, I=64, E=8, k=2,
                                wfmt="affine4", seed=113),
    # relu^2 experts on rows with a NaN, +inf or -inf input (bloomery PR #235:
    # relu^2 keeps a non-finite input non-finite), with a shared expert
    "mid_relu2_nonfinite": Workload("mid_relu2_nonfinite", T=160, H=256, I=192, E=16, k=4,
                                    act="relu2", rsf=2.5, I_shared=128, seed=114,
                                    nan_rows=(1, 90), posinf_rows=(3, 100), neginf_rows=(5, 150),
                                    tie_col=11),
    # Shared experts a whole number of routed widths wide (I_shared = m I):
    # at prompt sizes they run as m plan segments inside the routed launches
    # (relu^2 m = 2 as in Nemotron-H; SwiGLU m = 3 with the input limit;
    # 4-bit routed experts beside a bf16 shared expert, m = 1).
    "mid_relu2_shared_seg": Workload("mid_relu2_shared_seg", T=300, H=256, I=192, E=16, k=4,
                                     act="relu2", rsf=2.5, I_shared=384, seed=116),
    "mid_swiglu_shared_seg3": Workload("mid_swiglu_shared_seg3", T=200, H=256, I=128, E=12, k=3,
                                       rsf=1.25, I_shared=384, swiglu_limit=7.0, x_std=8.0,
                                       seed=117),
    "mid_affine4_shared_seg": Workload("mid_affine4_shared_seg", T=200, H=256, I=128, E=8, k=2,
                                       wfmt="affine4", I_shared=128, seed=118),
    # Block-FP8 e4m3 experts, one fp32 scale per 128 x 128 block (TensorFold
    # issue #548: the block-FP8 experts of the CUDA branches), with a
    # SwiGLU shared expert.
    "mid_fp8": Workload("mid_fp8", T=500, H=384, I=256, E=16, k=4, wfmt="fp8", scale_lo=1e-4,
                        scale_hi=3e-4, I_shared=128, seed=109),
    # relu^2 block-FP8 experts, with e4m3 NaN codes (S.1111.111) in three
    # down rows: the tokens routed to those experts get NaN in that column
    "mid_fp8_relu2": Workload("mid_fp8_relu2", T=200, H=256, I=384, E=24, k=6, act="relu2",
                              wfmt="fp8", rsf=2.5, scale_lo=1e-4, scale_hi=3e-4, seed=110,
                              fp8_nan=((0, 5), (3, 100), (7, 200))),
    # Block-FP8 codes over a wide range (exponent field N(7, 1.5), scales
    # 0.01-0.03): weights from about 1e-4 to 13, whose products reach far
    # past the bulk; the shapes of mid_fp8.
    "mid_fp8_wide": Workload("mid_fp8_wide", T=500, H=384, I=256, E=16, k=4, wfmt="fp8",
                             scale_lo=0.01, scale_hi=0.03, fp8_exp_mu=7.0, fp8_exp_sd=1.5,
                             I_shared=128, seed=115),
    # NVFP4 experts (TensorFold issue #548, the core/quant split: ModelOpt
    # NVFP4, uint8 [N, K/2], an e4m3 scale every 16 inputs, a global scale),
    # with a bf16 SwiGLU shared expert, and relu^2 NVFP4 experts.
    "mid_nvfp4": Workload("mid_nvfp4", T=300, H=384, I=256, E=16, k=4, wfmt="nvfp4",
                          I_shared=128, seed=119),
    "mid_nvfp4_relu2": Workload("mid_nvfp4_relu2", T=200, H=256, I=384, E=24, k=6, act="relu2",
                                wfmt="nvfp4", rsf=2.5, seed=120),
    # MXFP4 experts (the OCP MX format: E2M1 codes, an E8M0 scale every 32
    # inputs), relu^2 with a NaN scale in two down rows, and SwiGLU with a
    # bf16 shared expert.
    "mid_mxfp4": Workload("mid_mxfp4", T=300, H=384, I=256, E=16, k=4, wfmt="mxfp4",
                          I_shared=128, seed=123),
    "mid_mxfp4_relu2": Workload("mid_mxfp4_relu2", T=200, H=256, I=384, E=24, k=6,
                                act="relu2", wfmt="mxfp4", rsf=2.5, seed=124,
                                mx_nan=((1, 7), (5, 130))),
    # The softmax router family (TensorFold issue #548, the consolidation
    # proposal), with NaN rows and exact ties, over 64 experts.
    # No expert bias (the family has none): every score of an all-zero row
    # is exactly 1/64, a 64-way tie.
    "mid_softmax": Workload("mid_softmax", T=400, H=256, I=192, E=64, k=6, score="softmax",
                            router_std=0.1, bias_lo=0.0, bias_hi=0.0, seed=107,
                            nan_rows=(3, 250), zero_rows=(11, 300), onehot_tie_row=99),
    # swiglu_limit 10 with the inputs scaled so that about 16 % of the gate
    # and 33 % of the up pre-activations clamp (TensorFold issue #548, the
    # GLM experts' untested paths); the shared expert clamps too.
    "mid_swiglu_limit": Workload("mid_swiglu_limit", T=300, H=512, I=256, E=16, k=4,
                                 swiglu_limit=10.0, x_std=22.0, router_std=0.001, I_shared=192,
                                 seed=108),
}


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------

# Full-size workloads beyond the five above, for the next formats: the
# LFM2-MoE shapes with block-FP8 experts, at prefill and decode sizes.
EXTRA = {
    "lfm2_fp8_prefill_t4096": Workload("lfm2_fp8_prefill_t4096", T=4096, H=2048, I=1792, E=32,
                                       k=4, wfmt="fp8", scale_lo=1e-4, scale_hi=3e-4, seed=111),
    "lfm2_nvfp4_prefill_t4096": Workload("lfm2_nvfp4_prefill_t4096", T=4096, H=2048, I=1792,
                                         E=32, k=4, wfmt="nvfp4", seed=121),
    "lfm2_nvfp4_decode_t8": Workload("lfm2_nvfp4_decode_t8", T=8, H=2048, I=1792, E=32, k=4,
                                     wfmt="nvfp4", seed=122, weight_seed=121),
    "lfm2_mxfp4_prefill_t4096": Workload("lfm2_mxfp4_prefill_t4096", T=4096, H=2048, I=1792,
                                         E=32, k=4, wfmt="mxfp4", seed=125),
    "lfm2_mxfp4_decode_t8": Workload("lfm2_mxfp4_decode_t8", T=8, H=2048, I=1792, E=32, k=4,
                                     wfmt="mxfp4", seed=126, weight_seed=125),
    "lfm2_fp8_decode_t8": Workload("lfm2_fp8_decode_t8", T=8, H=2048, I=1792, E=32, k=4,
                                   wfmt="fp8", scale_lo=1e-4, scale_hi=3e-4, seed=112,
                                   weight_seed=111),
    # The decode step on the 4-bit weights: with the +2.0 boost as configured
    # (every token picks the four boosted experts), and without it (the same
    # expert weights and base bias, so the picks spread over the experts).
    "affine4_decode_t8": Workload("affine4_decode_t8", T=8, H=2048, I=1792, E=32, k=4,
                                  wfmt="affine4", seed=5, weight_seed=4, boost=2.0,
                                  boosted=(3, 11, 19, 27)),
    "affine4_flat_decode_t8": Workload("affine4_flat_decode_t8", T=8, H=2048, I=1792, E=32,
                                       k=4, wfmt="affine4", seed=5, weight_seed=4),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); NaN -> 0x7FC0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        v *= np.float32(std)
        out[s:s + m] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = rng.standard_normal(m, dtype=np.float32) * np.float32(std)
    return out.reshape(shape)


def _uniform_f32(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        u = rng.random(m, dtype=np.float32)
        out[s:s + m] = np.float32(lo) + np.float32(hi - lo) * u
    return out.reshape(shape)


def _words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform 32-bit words: each of the 8 nibbles is uniform on 0..15."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint32)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = rng.integers(0, 1 << 32, size=m, dtype=np.uint32)
    return out.reshape(shape)


def _fp8_codes(rng: np.random.Generator, shape, mu: float = 13.0, sd: float = 1.0) -> np.ndarray:
    """OCP FP8 E4M3 bytes drawn field by field, shaped like weights quantized
    with a per-block absmax scale (by default the block's largest weight
    near code 448, the bulk a few octaves below): sign uniform, exponent
    field round(N(mu, sd)) clipped to 0..15, mantissa uniform on 0..7; the
    NaN pattern S.1111.111 is replaced by S.1111.110 (448)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    mu32, sd32 = np.float32(mu), np.float32(sd)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        e = np.clip(np.rint(rng.standard_normal(m, dtype=np.float32) * sd32 + mu32), 0, 15)
        e = e.astype(np.uint8)
        mant = rng.integers(0, 8, size=m, dtype=np.uint8)
        sign = rng.integers(0, 2, size=m, dtype=np.uint8)
        mant[(e == 15) & (mant == 7)] = 6
        out[s:s + m] = (sign << 7) | (e << 3) | mant
    return out.reshape(shape)


def _bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = rng.integers(0, 256, size=m, dtype=np.uint8)
    return out.reshape(shape)


def _e4m3_scales(rng: np.random.Generator, shape, mu: float, sd: float) -> np.ndarray:
    """Positive OCP E4M3 scale codes: exponent field round(N(mu, sd))
    clipped to 0..15, mantissa uniform, never the NaN pattern."""
    n = int(np.prod(shape))
    e = np.clip(np.rint(rng.standard_normal(n, dtype=np.float32) * np.float32(sd) +
                        np.float32(mu)), 0, 15).astype(np.uint8)
    mant = rng.integers(0, 8, size=n, dtype=np.uint8)
    mant[(e == 15) & (mant == 7)] = 6
    return ((e << 3) | mant).reshape(shape)


def _children(seed: int):
    return [np.random.default_rng(c) for c in np.random.SeedSequence([0x5EED, seed]).spawn(10)]


def generate(wl: Workload, need_x: bool = True, experts: bool = True) -> dict:
    """Draw every input of ``wl``.

    Returns a dict of C-contiguous NumPy arrays. bf16 tensors are uint16 bit
    patterns. Keys: x [T,H] bf16, router_w [E,H] f32, bias [E] f32, and
    for bf16 experts w_up [E,n_up,H], w_down [E,H,I] bf16; for affine-4
    experts w_up (uint32 codes [E,n_up,H/8]), w_up_scales / w_up_biases
    (bf16 [E,n_up,H/64]) and the same three for w_down ([E,H,I/8],
    [E,H,I/64]); shared_up [I_s,H] and shared_down [H,I_s] bf16 when
    I_shared > 0 (shared_up is [2*I_s,H], gate rows first, for SwiGLU).
    With experts=False only x, router_w and bias are drawn (each tensor has
    its own stream, so the others are unchanged).
    """
    E, H, I, T = wl.E, wl.H, wl.I, wl.T
    xs = _children(wl.seed)
    ws = _children(wl.weight_seed if wl.weight_seed is not None else wl.seed)
    (c_x, c_wr, c_b, c_up, c_down, c_su, c_sd, c_codes, c_scales, c_qb) = range(10)
    out = {}
    if need_x:
        out["x"] = _normal_bf16(xs[c_x], (T, H), wl.x_std)
    out["router_w"] = _normal_f32(ws[c_wr], (E, H), wl.router_std)
    out["bias"] = _uniform_f32(ws[c_b], (E,), wl.bias_lo, wl.bias_hi)
    if wl.boost:
        for e in wl.boosted:
            out["bias"][e] = np.float32(out["bias"][e] + np.float32(wl.boost))
    n_up = wl.n_up
    if not experts:
        _construct_special_rows(wl, out)
        return out
    if wl.wfmt == "bf16":
        out["w_up"] = _normal_bf16(ws[c_up], (E, n_up, H), wl.w_std)
        out["w_down"] = _normal_bf16(ws[c_down], (E, H, I), wl.w_std)
    elif wl.wfmt == "affine4":
        g = wl.group
        out["w_up"] = _words(ws[c_codes], (E, n_up, H // 8))
        out["w_down"] = _words(ws[c_codes], (E, H, I // 8))
        out["w_up_scales"] = f32_to_bf16_bits(_uniform_f32(ws[c_scales], (E, n_up, H // g),
                                                           wl.scale_lo, wl.scale_hi))
        out["w_down_scales"] = f32_to_bf16_bits(_uniform_f32(ws[c_scales], (E, H, I // g),
                                                             wl.scale_lo, wl.scale_hi))
        out["w_up_biases"] = f32_to_bf16_bits(_uniform_f32(ws[c_qb], (E, n_up, H // g),
                                                           wl.qbias_lo, wl.qbias_hi))
        out["w_down_biases"] = f32_to_bf16_bits(_uniform_f32(ws[c_qb], (E, H, I // g),
                                                             wl.qbias_lo, wl.qbias_hi))
    elif wl.wfmt == "nvfp4":
        # codes: two uniform E2M1 codes per byte; per 16 inputs an E4M3 scale
        # drawn like absmax-scaled blocks (near 448 by default); per expert
        # matrix a global scale
        out["w_up"] = _bytes(ws[c_codes], (E, n_up, H // 2))
        out["w_down"] = _bytes(ws[c_codes], (E, H, I // 2))
        out["w_up_scales"] = _e4m3_scales(ws[c_scales], (E, n_up, H // 16), wl.fp8_exp_mu,
                                          wl.fp8_exp_sd)
        out["w_down_scales"] = _e4m3_scales(ws[c_scales], (E, H, I // 16), wl.fp8_exp_mu,
                                            wl.fp8_exp_sd)
        out["w_up_global"] = _uniform_f32(ws[c_qb], (E,), wl.global_lo, wl.global_hi)
        out["w_down_global"] = _uniform_f32(ws[c_qb], (E,), wl.global_lo, wl.global_hi)
    elif wl.wfmt == "mxfp4":
        # codes as NVFP4; per 32 inputs an E8M0 scale 2^(b - 127)
        out["w_up"] = _bytes(ws[c_codes], (E, n_up, H // 2))
        out["w_down"] = _bytes(ws[c_codes], (E, H, I // 2))

        def e8m0(rng, shape):
            n = int(np.prod(shape))
            b = np.rint(rng.standard_normal(n, dtype=np.float32) * np.float32(wl.mx_exp_sd) +
                        np.float32(wl.mx_exp_mu))
            return np.clip(b, 1, 254).astype(np.uint8).reshape(shape)
        out["w_up_scales"] = e8m0(ws[c_scales], (E, n_up, H // 32))
        out["w_down_scales"] = e8m0(ws[c_scales], (E, H, I // 32))
        for e, h in wl.mx_nan:
            out["w_down_scales"][e, h, (3 * h + e) % (I // 32)] = 0xFF
    elif wl.wfmt == "fp8":
        mu, sd = wl.fp8_exp_mu, wl.fp8_exp_sd
        out["w_up"] = _fp8_codes(ws[c_codes], (E, n_up, H), mu, sd)
        out["w_down"] = _fp8_codes(ws[c_codes], (E, H, I), mu, sd)
        for i, (e, h) in enumerate(wl.fp8_nan):
            # one NaN code per listed down row, alternating sign
            out["w_down"][e, h, (7 * h + e) % I] = 0x7F if i % 2 == 0 else 0xFF
        out["w_up_scales"] = _uniform_f32(ws[c_scales], (E, n_up // 128, H // 128),
                                          wl.scale_lo, wl.scale_hi)
        out["w_down_scales"] = _uniform_f32(ws[c_scales], (E, H // 128, I // 128),
                                            wl.scale_lo, wl.scale_hi)
    else:
        raise ValueError(f"unknown weight format {wl.wfmt!r}")
    if wl.I_shared:
        n_sup = 2 * wl.I_shared if wl.act == "swiglu" else wl.I_shared
        out["shared_up"] = _normal_bf16(ws[c_su], (n_sup, H), wl.w_std)
        out["shared_down"] = _normal_bf16(ws[c_sd], (H, wl.I_shared), wl.w_std)
    _construct_special_rows(wl, out)
    return out


def _construct_special_rows(wl: Workload, out: dict) -> None:
    """Rows whose routing is fixed by exact arithmetic, not by rounding.

    * NaN rows: every x entry is a bf16 NaN, so every router logit is NaN.
    * Zero rows: every x entry is 0, so every router logit is +0.
    * +inf / -inf rows: x has +inf (-inf) at column tie_col, so a logit is
      +inf or -inf by the sign of that router weight.
    * Zero tie row: x is all zeros, so every logit is +0 and every score
      the same; the bias of experts 1, 4, 6 is set to 0.125, above every
      other bias, which makes a three-way tie at the top.
    * One-hot tie row: x has a single 1.0 at column tie_col, and router
      weights (2, tie_col) and (5, tie_col) are both 2.0, with bias[5] set
      to bias[2], so experts 2 and 5 tie above the rest.
    The edits to the router weight and bias change other rows' routing too;
    they are part of the workload's definition.
    """
    x = out.get("x")
    if x is not None:
        for r in wl.nan_rows:
            x[r, :] = BF16_NAN
        for r in wl.zero_rows:
            x[r, :] = 0
        for r in wl.posinf_rows:
            x[r, wl.tie_col] = 0x7F80
        for r in wl.neginf_rows:
            x[r, wl.tie_col] = 0xFF80
    if wl.zero_tie_row is not None:
        if x is not None:
            x[wl.zero_tie_row, :] = 0
        for e in (1, 4, 6):
            if e < wl.E:
                out["bias"][e] = np.float32(0.125)
    if wl.onehot_tie_row is not None and wl.E > 5:
        if x is not None:
            x[wl.onehot_tie_row, :] = 0
            x[wl.onehot_tie_row, wl.tie_col] = BF16_ONE
        out["router_w"][2, wl.tie_col] = np.float32(2.0)
        out["router_w"][5, wl.tie_col] = np.float32(2.0)
        out["bias"][5] = out["bias"][2]


def slice_order_inputs(T: int, H: int, E: int) -> dict:
    """Router inputs whose top experts depend on how the logit is summed.

    x[t, h] = 2^(t % 3) for every h (a power of two: every product and sum
    below scales exactly), bias 0. Expert e's router row is zero except for
    one pattern, chosen by e % 4 and placed at slice m_e (slices of 64 h;
    m_e spread over H / 64 - 4 positions), with b = 2^24:
      0: w[64m + 63] = b, w[64m + 64] = 1, w[64m + 65] = -b   (across a slice end)
      1: w[64m + 31] = b, w[64m + 32] = 1, w[64m + 33] = -b   (inside one slice)
      2: w[64m] = b, w[64(m+1)] = 1, w[64(m+2)] = 1, w[64(m+3)] = -b
      3: w[5] = 0.5
    Needs H >= 256 and H % 64 == 0. Returns x (bf16 bits), router_w, bias and
    the pattern of each expert."""
    assert H >= 256 and H % 64 == 0
    b = np.float32(2.0 ** 24)
    wr = np.zeros((E, H), np.float32)
    n = H // 64 - 4
    pattern = np.arange(E) % 4
    for e in range(E):
        m = (e * 7 + 3) % (n + 1)
        p = pattern[e]
        if p == 0:
            wr[e, 64 * m + 63], wr[e, 64 * m + 64], wr[e, 64 * m + 65] = b, 1, -b
        elif p == 1:
            wr[e, 64 * m + 31], wr[e, 64 * m + 32], wr[e, 64 * m + 33] = b, 1, -b
        elif p == 2:
            wr[e, 64 * m], wr[e, 64 * (m + 1)], wr[e, 64 * (m + 2)], wr[e, 64 * (m + 3)] = b, 1, 1, -b
        else:
            wr[e, 5] = 0.5
    x = np.empty((T, H), np.uint16)
    for t in range(T):
        x[t, :] = f32_to_bf16_bits(np.full(1, 2.0 ** (t % 3), np.float32))[0]
    return {"x": x, "router_w": wr, "bias": np.zeros(E, np.float32), "pattern": pattern}


def _grid_bf16(rng: np.random.Generator, shape, lo: float, hi: float,
               signed: bool = True) -> np.ndarray:
    """bf16 bits of magnitudes drawn uniformly in [lo, hi) (never zero), with
    a uniform random sign when signed."""
    v = _uniform_f32(rng, shape, lo, hi)
    if signed:
        v = np.where(rng.integers(0, 2, size=v.shape) == 1, -v, v).astype(np.float32)
    return f32_to_bf16_bits(v)


def exact_inputs(wl: Workload, nonfinite: bool = False) -> dict:
    """Inputs on which every expert projection has at most one non-zero
    term, so a projection's value is one product of two bf16 numbers (exact
    in fp32) whatever order a kernel sums in. What is left to pin bit for bit
    is then the engine's own fp32 order: the activation epilogue and its one
    rounding to bf16, and the combine.

    * x: token t is one-hot, 1.0 at column onehot_col(t) = (37 t) mod H.
    * router weight N(0, 0.5) fp32 and expert bias U(bias_lo, bias_hi), so
      the logit of expert e is its router weight at the token's column.
    * up weights (relu^2 and the up half of gate_up): magnitudes U[0.25, 4)
      with random signs; SwiGLU gate rows: U[24, 64), where the fp32 sigmoid
      is exactly 1, so silu(g) u is the fp32 product g u.
    * down weights: row n of expert e has one non-zero, at column
      (7 n + 3 e) mod I, magnitude U[0.25, 4) with a random sign. The shared
      expert is built the same way (as expert E).
    * nonfinite (relu^2 only): up weight (e, n, c) set to -inf for e = 1,
      +inf for e = 2 and NaN for e = 3, with n = 5 and c the column of token
      e; the router weight of expert e at that column is set to 10, so that
      token (and every token sharing its column) picks expert e first. A
      token routed to such an expert from another column multiplies the
      non-finite weight by 0 (NaN); the token on the column gets -inf, +inf
      or NaN as its pre-activation.
    Draws come from SeedSequence([0x5EED, 0xB17, seed]) children in the
    order x-free: router, bias, up, down, shared up, shared down."""
    E, H, I, T = wl.E, wl.H, wl.I, wl.T
    rr, rb, ru, rd, rsu, rsd = [np.random.default_rng(c) for c in
                                np.random.SeedSequence([0x5EED, 0xB17, wl.seed]).spawn(6)]
    out = {}
    x = np.zeros((T, H), np.uint16)
    x[np.arange(T), onehot_col(np.arange(T), H)] = BF16_ONE
    out["x"] = x
    out["router_w"] = _normal_f32(rr, (E, H), 0.5)
    out["bias"] = _uniform_f32(rb, (E,), wl.bias_lo, wl.bias_hi)

    def up_rows(rng, experts, n_rows, I_):
        if wl.act == "swiglu":
            gate = _grid_bf16(rng, (experts, I_, H), 24.0, 64.0, signed=False)
            up = _grid_bf16(rng, (experts, I_, H), 0.25, 4.0)
            return np.concatenate([gate, up], axis=1)
        return _grid_bf16(rng, (experts, n_rows, H), 0.25, 4.0)

    def down_rows(rng, experts, I_, e0=0):
        d = np.zeros((experts, H, I_), np.uint16)
        vals = _grid_bf16(rng, (experts, H), 0.25, 4.0)
        n = np.arange(H)
        for e in range(experts):
            d[e, n, (7 * n + 3 * (e0 + e)) % I_] = vals[e]
        return d

    out["w_up"] = up_rows(ru, E, wl.n_up, I)
    out["w_down"] = down_rows(rd, E, I)
    if wl.I_shared:
        n_sup = 2 * wl.I_shared if wl.act == "swiglu" else wl.I_shared
        out["shared_up"] = up_rows(rsu, 1, n_sup, wl.I_shared)[0]
        out["shared_down"] = down_rows(rsd, 1, wl.I_shared, e0=E)[0]
    if nonfinite:
        assert wl.act == "relu2" and E > 3 and T > 3
        bits = {1: 0xFF80, 2: 0x7F80, 3: BF16_NAN}      # -inf, +inf, NaN
        for e, b in bits.items():
            c = onehot_col(e, H)
            out["w_up"][e, 5, c] = b
            out["router_w"][e, c] = np.float32(10.0)
    return out


def onehot_col(t, H: int):
    """Column of the single 1.0 of token t in exact_inputs."""
    return (37 * np.asarray(t)) % H


def norm_inputs(T: int, H: int, seed: int = 0, with_h: bool = True) -> dict:
    """Inputs of the fused residual add + RMSNorm before the block: h and
    residual [T,H] bf16 ~ N(0, 1), gamma [H] bf16 ~ N(1, 0.1) (a trained
    norm scale stays near 1), eps 1e-5. Drawn from
    SeedSequence([0x5EED, 0x4E0, seed]) children in the order h, residual,
    gamma."""
    rh, rr, rg = [np.random.default_rng(c)
                  for c in np.random.SeedSequence([0x5EED, 0x4E0, seed]).spawn(3)]
    out = {"residual": _normal_bf16(rr, (T, H), 1.0), "eps": 1e-5}
    out["h"] = _normal_bf16(rh, (T, H), 1.0) if with_h else None
    g = rg.standard_normal(H, dtype=np.float32) * np.float32(0.1) + np.float32(1.0)
    out["gamma"] = f32_to_bf16_bits(g)
    return out


def by_name(name: str) -> Workload:
    for w in CONFIGS:
        if w.name == name:
            return w
    if name in MID:
        return MID[name]
    if name in EXTRA:
        return EXTRA[name]
    raise KeyError(name)
