"""One family of bits at every row count.

TensorFold issue #548 (the kernel registry in the core/quant split) asks
that a row's bits never depend on how many rows share a launch. With the
row_invariant option every batch takes the MFMA tiles, whose sums for one
token row use the same K order and the same epilogue whatever the other rows
of the tile are (padding rows read as zeros, 128- and 256-row tiles walk K
alike), and the router already adds the same K slices at every row count.
Each case runs the first T tokens of one workload for T = the workload's
size, 100, 8 and 1 and requires every token's fp32 and bf16 output rows to
be the same bits in every call, NaN in the same places. Without the option
the decode-sized calls take the weight-streaming form, and the bf16 case
checks that their bits then differ: the equality is the option's doing.
"""
import numpy as np
import pytest
import torch

from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
CASES = ["lfm2_prefill_t4096", "mid_relu2_shared", "mid_affine4", "mid_fp8", "mid_swiglu_limit",
         "mid_relu2_nonfinite", "mid_relu2_shared_seg", "mid_nvfp4", "mid_mxfp4"]


def _run(wl, inp, T, row_invariant):
    block = lib.block_from_arrays(wl, inp)
    block.row_invariant = row_invariant
    x = lib.x_to_device(np.ascontiguousarray(inp["x"][:T]))
    out32 = torch.empty((T, wl.H), dtype=torch.float32, device=DEV).fill_(float("nan"))
    block.forward(x, out_dtype=torch.float32, out=out32)
    out16 = block.forward(x)
    torch.cuda.synchronize()
    return out32.cpu().numpy(), out16.view(torch.int16).cpu().numpy().view(np.uint16)


def _same_bits(a, b):
    nan = np.isnan(a)
    assert (np.isnan(b) == nan).all()
    return (a[~nan].view(np.uint32) == b[~nan].view(np.uint32)).all()


@pytest.mark.parametrize("name", CASES)
def test_token_bits_do_not_depend_on_the_row_count(name):
    wl = W.by_name(name)
    inp = W.generate(wl)
    full32, full16 = _run(wl, inp, wl.T, True)
    for T in (100, 8, 1):
        o32, o16 = _run(wl, inp, T, True)
        assert _same_bits(o32, full32[:T]), (name, T)
        assert (o16 == full16[:T]).all(), (name, T)
    if name == "lfm2_prefill_t4096":
        s32, _ = _run(wl, inp, 8, False)
        assert not _same_bits(s32, full32[:8])
