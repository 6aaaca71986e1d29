"""Tile-packed expert weights (moe_pack_tiles) on the GPU.

The packed copy is a permutation of the caller's bf16 expert weights (or
block-FP8 codes) that
the MFMA tiles read in place of them: a stage then holds the same values as
without it, so every output must be the same bits, fp32 and bf16. The layout
itself is checked against the header's description, derived again here with
NumPy. Zeroing the copy after the first call shows which calls read it: the
prompt-sized tiles (and row_invariant batches) must change, the decode form
must not.
"""
import numpy as np
import pytest
import torch

from sigmoid_top_routing_amd import lib
from sigmoid_top_routing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def packed_reference(w, gate_up, I):
    """tiles[e][nt][ks][s] as include/moe.h states it, from w [E, N, K]:
    uint16 (bf16, 8 per slot) or uint8 (FP8 codes, 16 per slot)."""
    E, N, K = w.shape
    nts = -(-I // 128) if gate_up else -(-N // 256)
    per = 16 // w.itemsize                      # weights per 16-byte slot
    spr = 32 // per                             # slots per row and K-slice
    s = np.arange(256 * spr)
    r = s // spr
    c = (s % spr) ^ ((r // 4) % 4) if spr == 4 else (s % 2) ^ ((r // 8) % 2)
    out = np.empty((E, nts, K // 32, 256 * spr, per), w.dtype)
    for nt in range(nts):
        if gate_up:
            n = np.minimum(128 * nt + r % 128, I - 1)
            row = np.where(r < 128, n, I + n)
        else:
            row = np.minimum(256 * nt + r, N - 1)
        for ks in range(K // 32):
            cols = 32 * ks + per * c[:, None] + np.arange(per)[None, :]
            out[:, nt, ks] = w[:, row[:, None], cols]
    return out.reshape(-1)


@pytest.mark.parametrize("act,E,H,I,wfmt", [("swiglu", 3, 128, 192, "bf16"),
                                            ("relu2", 2, 320, 192, "bf16"),
                                            ("swiglu", 2, 256, 256, "bf16"),
                                            ("swiglu", 3, 128, 384, "fp8"),
                                            ("relu2", 2, 384, 128, "fp8")])
def test_pack_layout(act, E, H, I, wfmt):
    rng = np.random.default_rng(7)
    d = lib.make_dims(0, H, I, E, 1, act=act, wfmt=wfmt)
    n_up = 2 * I if act == "swiglu" else I
    dt = np.uint16 if wfmt == "bf16" else np.uint8
    for which, shape, gate_up in (("up", (E, n_up, H), act == "swiglu"),
                                  ("down", (E, H, I), False)):
        w = rng.integers(0, np.iinfo(dt).max + 1, size=shape, dtype=dt)   # any bits, NaNs included
        wt = torch.from_numpy(w.view(np.uint8)).to(DEV)
        tiles = lib.pack_tiles(d, which, wt)
        torch.cuda.synchronize()
        got = tiles.cpu().numpy().view(dt)
        want = packed_reference(w, gate_up, I)
        assert got.shape == want.shape and (got == want).all(), which


def bits(t):
    t = t.cpu()
    return (t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)).numpy()


def outputs(blk, x, T, H):
    res = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((T, H), float("nan"), dtype=dt, device=DEV)
        ids = torch.full((T, blk.k), -1, dtype=torch.int32, device=DEV)
        blk.forward(x, out_dtype=dt, out=out, ids_out=ids)
        torch.cuda.synchronize()
        res[dt] = (bits(out), ids.cpu().numpy())
    return res


def same(a, b):
    return all((a[dt][0] == b[dt][0]).all() and (a[dt][1] == b[dt][1]).all() for dt in a)


CASES = [("lfm2_prefill_t4096", False), ("mid_swiglu", False), ("mid_swiglu_bigseg", False),
         ("mid_relu2_shared", False), ("mid_relu2_shared_seg", False),
         ("mid_swiglu_limit", False), ("mid_e256_k8", False), ("mid_nan_ties", False),
         ("mid_relu2_nonfinite", False), ("lfm2_decode_t8", True), ("mid_swiglu", True),
         ("mid_fp8", False), ("mid_fp8_relu2", False), ("mid_fp8_wide", False),
         ("lfm2_fp8_prefill_t4096", False), ("lfm2_fp8_decode_t8", True)]


@pytest.mark.parametrize("name,row_invariant", CASES)
def test_forward_with_tiles_gives_the_same_bits(name, row_invariant):
    wl = W.by_name(name)
    inp = W.generate(wl)
    blk = lib.block_from_arrays(wl, inp)
    blk.row_invariant = row_invariant
    x = lib.x_to_device(inp["x"])
    plain = outputs(blk, x, wl.T, wl.H)
    blk.pack_tiles()
    torch.cuda.synchronize()
    packed = outputs(blk, x, wl.T, wl.H)
    assert same(plain, packed)
    # the tiles read the copy: zeroed, the routed sums change
    blk.w_up_tiles.zero_()
    blk.w_down_tiles.zero_()
    zeroed = outputs(blk, x, wl.T, wl.H)
    assert not same(plain, zeroed)


@pytest.mark.parametrize("name", ["lfm2_decode_t8", "lfm2_fp8_decode_t8"])
def test_decode_form_reads_the_callers_weights(name):
    # T * k <= 2 E without row_invariant: the weight-streaming form, which
    # reads w_up / w_down as stored whatever copy is given
    wl = W.by_name(name)
    inp = W.generate(wl)
    blk = lib.block_from_arrays(wl, inp)
    x = lib.x_to_device(inp["x"])
    plain = outputs(blk, x, wl.T, wl.H)
    blk.pack_tiles()
    blk.w_up_tiles.zero_()
    blk.w_down_tiles.zero_()
    assert same(plain, outputs(blk, x, wl.T, wl.H))
