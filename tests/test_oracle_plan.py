"""Pins of the oracle's expert plan (histogram, exclusive scan, stable
permutation into per-expert segments), against Python's own stable sort.

The plan is the grouped expert plan of TensorFold issue #548 ("One grouped-
MoE layer: the routing plan plus per-format expert kernels"); the order
inside a segment (ascending assignment index) is this project's reading.
"""
import numpy as np
import pytest

import oracle
from sigmoid_top_routing_amd import workloads as W


def _check(ids, E):
    T, k = ids.shape
    A = T * k
    counts, offsets, srt, slot = oracle.plan(ids, E)
    flat = [int(v) for v in ids.reshape(-1)]
    expect = sorted(range(A), key=lambda a: (flat[a], a))     # Python's stable sort
    assert list(srt) == expect
    assert list(counts) == [flat.count(e) for e in range(E)]
    assert offsets[0] == 0 and offsets[E] == A
    assert list(np.diff(offsets)) == list(counts)
    assert (slot[srt] == np.arange(A)).all()
    for e in range(E):
        seg = srt[offsets[e]:offsets[e + 1]]
        assert all(flat[a] == e for a in seg)


@pytest.mark.parametrize("name", ["tiny_t64_e8_k2", "mid_nan_ties", "mid_e256_k8", "mid_swiglu"])
def test_plan_of_routed_workloads(name):
    wl = W.by_name(name)
    inp = W.generate(wl)
    ids, _ = oracle.route(inp["x"], inp["router_w"], inp["bias"], wl.k)
    _check(ids, wl.E)


def test_plan_random_and_degenerate_ids():
    rng = np.random.default_rng(3)
    for T, k, E in ((1, 1, 1), (5, 3, 4), (100, 4, 32), (37, 8, 256)):
        _check(rng.integers(0, E, size=(T, k)).astype(np.int32), E)
    # every assignment on one expert; all other segments empty
    _check(np.full((50, 1), 3, np.int32), 8)
    # empty input
    counts, offsets, srt, slot = oracle.plan(np.zeros((0, 2), np.int32), 4)
    assert (counts == 0).all() and (offsets == 0).all() and srt.size == 0
