"""moe_forward_noalloc against moe_forward on the GPU (through the C ABI).

The no-allocation entry point runs the same kernels with its workspace in
the library's static device scratch, which keeps the last call's contents:
two or three calls in a row, each smaller than the one before, must each
give exactly the bytes moe_forward gives with a fresh workspace (ids,
weights, plan offsets and output; bf16 and fp32 outputs).
"""
import numpy as np
import pytest
import torch

from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _call(block, x, dt, noalloc):
    T = x.shape[0]
    out = torch.full((T, block.H), float("nan"), dtype=dt, device=DEV)
    ids = torch.full((T, block.k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, block.k), float("nan"), dtype=torch.float32, device=DEV)
    offs = torch.full((block.E + 1,), -7, dtype=torch.int32, device=DEV)
    if noalloc:
        block.forward_noalloc(x, out_dtype=dt, out=out, ids_out=ids, weights_out=w,
                              offsets_out=offs)
    else:
        ws = torch.full((lib.workspace_bytes(block.dims(T, dt)),), 0xA5, dtype=torch.uint8,
                        device=DEV)
        block.forward(x, out_dtype=dt, out=out, ids_out=ids, weights_out=w, offsets_out=offs,
                      workspace=ws)
    torch.cuda.synchronize()
    return [t.view(torch.uint8).cpu().numpy() for t in (out, ids, w, offs)]


@pytest.mark.parametrize("name,Ts", [
    ("mid_relu2_shared", (300, 120, 8)),     # shared expert, rsf 2.5; the last call decode-sized
    ("mid_swiglu", (600, 7)),
    ("mid_affine4", (256, 8)),               # 4-bit: decoded weights in the scratch, then the staged decode
    ("lfm2_prefill_t4096", (1024, 8)),       # LFM2 shapes, 48 MB of scratch, then the decode step
])
def test_noalloc_matches_forward(name, Ts):
    wl = W.by_name(name)
    inp = W.generate(wl.with_(T=Ts[0]) if wl.T < Ts[0] else wl)
    block = lib.block_from_arrays(wl, inp)
    for i, T in enumerate(Ts):
        assert lib.workspace_bytes(block.dims(T, torch.float32)) <= lib.NOALLOC_SCRATCH_BYTES
        x = lib.x_to_device(np.ascontiguousarray(inp["x"][:T]))
        dt = torch.float32 if i % 2 else torch.bfloat16
        got = _call(block, x, dt, noalloc=True)
        want = _call(block, x, dt, noalloc=False)
        for g, w_, what in zip(got, want, ("out", "ids", "weights", "offsets")):
            assert (g == w_).all(), f"{name} T={T}: {what} differs"
