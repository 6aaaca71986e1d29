"""Bit-for-bit pins of the engine's own fp32 order on the GPU.

The pages pin the combine bitwise, not by tolerance: folding the routed
scale into each expert weight survived every tolerance-based case and was
caught only on data that separates the two forms (vllm.cpp PR #684, the
review-repairs commit; the W2 commit fixes the order: the routed scale
multiplies the finished routed sum, the shared output is added untouched;
relu^2 and silu * up widen to fp32 and round once).

On inputs where every expert projection is a single exact product
(workloads.exact_inputs: one-hot tokens, one non-zero per down row) the
only arithmetic left whose bits depend on the implementation is the
activation epilogue with its rounding to bf16 and the combine. The fp32
output of moe_forward must then equal the oracle's fp32 mimic
(oracle.combine32 over oracle.expert_rows32) in every bit, NaN in the same
places, at prompt sizes (the MFMA tiles) and decode sizes (the streaming
kernel). Each case first asserts that its data separates the engine's form
from the folded one, so a kernel that folded the scale turns the test red.
"""
import numpy as np
import pytest
import torch

import oracle
from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"

# name: (workload, non-finite up weights, Laguna's fold of the routed scale)
CASES = {
    # relu^2 experts, routed scale 2.5, a relu^2 shared expert
    "relu2_shared": (W.Workload("pin_relu2", T=300, H=256, I=192, E=16, k=4, act="relu2",
                                rsf=2.5, I_shared=128, bias_lo=-0.1, bias_hi=0.1, seed=500),
                     False, False),
    # SwiGLU with saturated gates, a decimal routed scale, a SwiGLU shared expert
    "swiglu_shared": (W.Workload("pin_swiglu", T=300, H=256, I=128, E=16, k=4, rsf=0.7,
                                 I_shared=64, bias_lo=-0.1, bias_hi=0.1, seed=501), False, False),
    # relu^2 of -inf, +inf and NaN pre-activations (and NaN from inf * 0)
    "relu2_nonfinite": (W.Workload("pin_relu2_nonfinite", T=300, H=256, I=192, E=16, k=4,
                                   act="relu2", rsf=1.5, bias_lo=-0.1, bias_hi=0.1, seed=502),
                        True, False),
    # relu^2 with a shared expert twice the routed width: at the prompt size
    # it runs as two plan segments whose partial rows the combine adds
    "relu2_shared_seg": (W.Workload("pin_relu2_seg", T=300, H=256, I=128, E=16, k=4,
                                    act="relu2", rsf=2.5, I_shared=256, bias_lo=-0.1,
                                    bias_hi=0.1, seed=504), False, False),
    # Laguna's fold (no shared expert): the scale inside each term, which
    # must then give the folded bits and not the engine's
    "swiglu_laguna_fold": (W.Workload("pin_swiglu_fold", T=300, H=256, I=128, E=16, k=4,
                                      rsf=2.5, bias_lo=-0.1, bias_hi=0.1, seed=503),
                           False, True),
}


def _bits_equal(got, want):
    """NaN in the same places, every other element the same 32 bits."""
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all(), np.argwhere(np.isnan(got) != nan)[:5]
    g, w = got[~nan].view(np.uint32), want[~nan].view(np.uint32)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{bad.size} elements differ, first: {got[~nan][bad[:4]]} vs {want[~nan][bad[:4]]}"


# (case, T): T None is the case's own prompt-sized batch; 8 and 1 take the
# decode form. One token of the non-finite case routes only to poisoned
# experts from another column (an all-NaN row, nothing left to separate).
RUNS = [(c, T) for c in sorted(CASES) for T in (None, 8, 1) if not (CASES[c][1] and T == 1)]


@pytest.mark.parametrize("case,T", RUNS)
def test_fp32_output_is_the_engine_order_bit_for_bit(case, T):
    wl, nonfinite, fold = CASES[case]
    inp = W.exact_inputs(wl, nonfinite=nonfinite)
    if T is not None:
        assert T * wl.k <= 2 * wl.E          # the decode form
        wl = wl.with_(T=T)
        inp = dict(inp, x=np.ascontiguousarray(inp["x"][:T]))
    block = lib.block_from_arrays(wl, inp)
    block.fold_routed_scale = fold
    x = lib.x_to_device(inp["x"])
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    out32 = torch.empty((wl.T, wl.H), dtype=torch.float32, device=DEV).fill_(float("nan"))
    block.forward(x, out_dtype=torch.float32, out=out32, ids_out=ids, weights_out=w)
    out16 = block.forward(x)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()

    ids_ref, w_ref = oracle.route(inp["x"], inp["router_w"], inp["bias"], wl.k)
    assert (ids == ids_ref).all()
    assert (np.abs(w - w_ref) <= 1e-6 * np.abs(w_ref)).all()

    toks = np.arange(wl.T)
    y, shared, inexact = oracle.expert_rows32(wl, inp, toks, ids)
    assert inexact == 0
    engine = oracle.combine32(w, y, shared, wl.rsf)
    folded = oracle.combine32(w, y, shared, wl.rsf, fold=True)
    want = folded if fold else engine
    fin = np.isfinite(engine) & np.isfinite(folded)
    sep = (engine[fin].view(np.uint32) != folded[fin].view(np.uint32)).mean()
    assert sep > 0.05, f"the data separates only {sep:.1%} of the elements"
    if nonfinite and T is None:
        assert np.isnan(want).any() and np.isinf(want).any() and np.isfinite(want).any()

    _bits_equal(out32.cpu().numpy(), want)
    # the bf16 output is the one rounding of the fp32 sum
    got16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    want16 = W.f32_to_bf16_bits(want)
    nan = np.isnan(want)
    assert (got16[~nan] == want16[~nan]).all()
    assert ((got16[nan] & 0x7FFF) > 0x7F80).all()
