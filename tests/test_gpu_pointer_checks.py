"""The boundary refuses host memory before any launch, also once the
library has cached the device allocations of earlier calls (it queries the
HIP runtime about a pointer only the first time it sees its allocation)."""
import numpy as np
import pytest
import torch

from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_host_memory_is_refused_before_and_after_cached_calls():
    wl = W.TINY
    inp = W.generate(wl)
    block = lib.block_from_arrays(wl, inp)
    x = lib.x_to_device(inp["x"])
    ref = block.forward(x)
    torch.cuda.synchronize()
    host = torch.from_numpy(inp["x"].view(np.int16).copy()).view(torch.bfloat16)
    pinned = host.pin_memory()
    for bad in (host, pinned):
        for _ in range(2):
            with pytest.raises(lib.MoeError, match="not device memory|not memory the HIP runtime"):
                block.forward(bad)
    # an output in host memory is refused too, and the device call still works
    with pytest.raises(lib.MoeError, match="not device memory|not memory the HIP runtime"):
        block.forward(x, out=torch.empty((wl.T, wl.H), dtype=torch.bfloat16).pin_memory())
    again = block.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
