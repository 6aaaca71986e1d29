"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and refuses bad arguments on the host before anything is enqueued
(no call here reaches a HIP launch)."""
import ctypes as C
import os
import re
import subprocess

import pytest
import torch

from sigmoid_top_routing_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*\*?\s*(moe_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = lib.load()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIBPATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def dims(**kw):
    base = dict(T=16, H=128, I=256, E=8, k=2)
    base.update(kw)
    return lib.make_dims(**base)


def status_of(fn):
    try:
        fn()
    except lib.MoeError as e:
        return e.code, str(e)
    return 0, ""


def ws_bytes(d):
    n = C.c_size_t()
    rc = lib.load().moe_workspace_bytes(C.byref(d), C.byref(n))
    return rc, n.value


def test_workspace_bytes_grows_with_the_problem():
    rc, small = ws_bytes(dims())
    assert rc == 0 and small > 0
    rc, big = ws_bytes(dims(T=4096, H=2048, I=1792, E=32, k=4))
    assert rc == 0 and big > 16384 * 2048 * 4
    rc, shared = ws_bytes(dims(I_shared=128))
    assert rc == 0 and shared > small


def test_workspace_bytes_past_4gib_of_down_rows():
    # T*k*H*4 = 4.59e9 bytes of per-assignment fp32 rows: the layout is in
    # size_t and the call is accepted (T*k*H stays below 2^31 elements)
    rc, n = ws_bytes(dims(T=140000, H=2048, I=128, E=8, k=4))
    assert rc == 0 and n > 140000 * 4 * 2048 * 4 > (1 << 32)


@pytest.mark.parametrize("bad,code,word", [
    (dict(H=100), -2, "H = 100"),
    (dict(H=0), -2, "H = 0"),
    (dict(I=96), -2, "I = 96"),
    (dict(E=0), -2, "E = 0"),
    (dict(E=300), -2, "E = 300"),
    (dict(k=3, E=2), -2, "k = 3"),
    (dict(k=9, E=16), -2, "k = 9"),
    (dict(T=-1), -2, "T = -1"),
    (dict(I_shared=100), -2, "I_shared = 100"),
])
def test_bad_shapes_are_refused(bad, code, word):
    rc, _ = ws_bytes(dims(**bad))
    assert rc == code
    assert word in lib.load().moe_last_error().decode()


def test_unsupported_options_are_refused():
    d = dims()
    d.act = 7
    assert ws_bytes(d)[0] == -4
    d = dims(wfmt="affine4")
    d.group = 32
    assert ws_bytes(d)[0] == -4
    assert "group = 32" in lib.load().moe_last_error().decode()
    d = dims()
    d.out_dtype = 5
    assert ws_bytes(d)[0] == -4
    d = dims()
    d.score_fn = 2
    assert ws_bytes(d)[0] == -4
    assert "score_fn = 2" in lib.load().moe_last_error().decode()
    d = dims(act="relu2", swiglu_limit=10.0)
    assert ws_bytes(d)[0] == -4
    assert "swiglu_limit" in lib.load().moe_last_error().decode()
    for bad in (-1.0, float("nan"), float("inf")):
        assert ws_bytes(dims(swiglu_limit=bad))[0] == -2
    assert ws_bytes(dims(swiglu_limit=10.0))[0] == 0
    # Laguna's fold of the routed scale: only without a shared expert
    assert ws_bytes(dims(fold_routed_scale=True))[0] == 0
    assert ws_bytes(dims(fold_routed_scale=True, I_shared=64))[0] == -4
    assert "shared expert" in lib.load().moe_last_error().decode()
    d = dims()
    d.fold_routed_scale = 2
    assert ws_bytes(d)[0] == -4
    # one family of bits at every row count: 0 or 1; with it a decode-sized
    # 4-bit batch decodes its experts to bf16 for the tiles
    d = dims()
    d.row_invariant = 2
    assert ws_bytes(d)[0] == -4
    assert "row_invariant" in lib.load().moe_last_error().decode()
    rc, n_stream = ws_bytes(dims(wfmt="affine4", T=8, H=256, I=256, E=8, k=2))
    rc1, n_tiles = ws_bytes(dims(wfmt="affine4", T=8, H=256, I=256, E=8, k=2, row_invariant=True))
    assert rc == rc1 == 0 and n_tiles >= n_stream + 8 * 512 * 256 * 2
    # NVFP4 and MXFP4: decode-sized batches stream the codes, prompt-sized
    # ones read them on the MFMA tiles: no decoded copy either way. With H
    # below 128 (too few K-slices for the tiles' ring) only decode sizes
    # are taken
    for fmt in ("nvfp4", "mxfp4"):
        for T in (8, 64):
            rc, nq = ws_bytes(dims(wfmt=fmt, T=T, H=256, I=256, E=8, k=2))
            rc16, n16 = ws_bytes(dims(T=T, H=256, I=256, E=8, k=2))
            assert rc == rc16 == 0 and nq == n16
        assert ws_bytes(dims(wfmt=fmt, T=8, H=64, I=256, E=8, k=2))[0] == 0
        assert ws_bytes(dims(wfmt=fmt, T=64, H=64, I=256, E=8, k=2))[0] == -4
        assert "H, I >= 128" in lib.load().moe_last_error().decode()
        d = dims(wfmt=fmt, T=8, H=64, I=256, E=8, k=2)
        d.row_invariant = 1
        assert ws_bytes(d)[0] == -4
    assert ws_bytes(dims(score="softmax"))[0] == 0
    assert ws_bytes(dims(wfmt="fp8", H=192))[0] == -2
    assert "multiples of 128" in lib.load().moe_last_error().decode()
    # FP8 codes are read at their stored width at prompt sizes (the MFMA
    # tiles) and at decode sizes (the stream): no more workspace than bf16.
    # Past 64 K-blocks (K > 8192) the tiles do not take them and a prompt-sized
    # batch holds the decoded weights of its experts.
    for T in (64, 8):
        rc, n8 = ws_bytes(dims(wfmt="fp8", T=T, H=256, I=256, E=8, k=2))
        rc16, n16 = ws_bytes(dims(T=T, H=256, I=256, E=8, k=2))
        assert rc == rc16 == 0 and n8 == n16
    rc, n8 = ws_bytes(dims(wfmt="fp8", T=64, H=8320, I=128, E=8, k=2))
    rc16, n16 = ws_bytes(dims(T=64, H=8320, I=128, E=8, k=2))
    assert rc == rc16 == 0 and n8 >= n16 + 8 * 256 * 8320 * 2     # eight experts decoded


def test_add_rmsnorm_refuses_bad_shapes_and_pointers():
    L = lib.load()
    f = L.moe_add_rmsnorm
    assert f(0, 2048, None, None, None, 1e-5, None, None, None) == 0     # nothing to do
    for T, H, eps, word in [(4, 100, 1e-5, "H = 100"), (4, 8256, 1e-5, "H = 8256"),
                            (-1, 64, 1e-5, "T = -1"), (4, 64, float("nan"), "eps")]:
        assert f(T, H, None, None, None, eps, None, None, None) == -2
        assert word in L.moe_last_error().decode()
    assert f(4, 64, None, None, None, 1e-5, None, None, None) == -1
    assert "residual is NULL" in L.moe_last_error().decode()
    assert f(4, 64, None, _fake(4096 + 8), _fake(4096), 1e-5, None, _fake(4096), None) == -3


def _fake(addr):
    return C.c_void_p(addr)


def test_forward_refuses_null_misaligned_and_short_workspace():
    L = lib.load()
    d = dims()
    w = lib.Weights()
    # NULL weights struct
    rc = L.moe_forward(C.byref(d), None, _fake(0x1000), _fake(0x1000), _fake(0x1000), 1 << 30,
                       None, None, None, None)
    assert rc == -1
    # a missing router weight
    rc = L.moe_forward(C.byref(d), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -1 and "router_w" in L.moe_last_error().decode()
    # a misaligned expert weight
    w = lib.Weights(router_w=0x1000, w_up=0x2008, w_down=0x3000)
    rc = L.moe_forward(C.byref(d), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -3 and "w_up" in L.moe_last_error().decode()
    # a short workspace
    w = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000)
    need = lib.workspace_bytes(d)
    rc = L.moe_forward(C.byref(d), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       need - 1, None, None, None, None)
    assert rc == -5 and str(need) in L.moe_last_error().decode()
    # 4-bit weights without scales
    da = dims(wfmt="affine4")
    rc = L.moe_forward(C.byref(da), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -1 and "scales" in L.moe_last_error().decode()
    # NVFP4 weights without their global scales
    dn = dims(wfmt="nvfp4")
    wn = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000, w_up_scales=0x4000,
                     w_down_scales=0x5000)
    rc = L.moe_forward(C.byref(dn), C.byref(wn), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -1 and "w_up_global" in L.moe_last_error().decode()
    # MXFP4 weights without their E8M0 scales
    dm = dims(wfmt="mxfp4")
    rc = L.moe_forward(C.byref(dm), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -1 and "w_up_scales" in L.moe_last_error().decode()
    # a shared expert without its weights
    ds = dims(I_shared=64)
    rc = L.moe_forward(C.byref(ds), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -1 and "shared_up" in L.moe_last_error().decode()


def test_noalloc_refuses_problems_past_its_scratch_before_any_launch():
    # moe_forward_noalloc takes its workspace from a static device array of
    # MOE_NOALLOC_SCRATCH_BYTES; a call that needs more is refused on the host
    L = lib.load()
    w = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000)
    big = dims(T=4096, H=2048, I=1792, E=32, k=4)
    assert lib.workspace_bytes(big) > lib.NOALLOC_SCRATCH_BYTES
    rc = L.moe_forward_noalloc(C.byref(big), C.byref(w), _fake(0x1000), _fake(0x1000), None,
                               None, None, None)
    msg = L.moe_last_error().decode()
    assert rc == -5 and "MOE_NOALLOC_SCRATCH_BYTES" in msg and str(lib.NOALLOC_SCRATCH_BYTES) in msg
    # 4-bit experts of a prompt-sized batch need room for their decoded weights
    q4 = dims(T=1024, H=2048, I=1792, E=32, k=4, wfmt="affine4")
    rc = L.moe_forward_noalloc(C.byref(q4), C.byref(w), _fake(0x1000), _fake(0x1000), None,
                               None, None, None)
    assert rc == -5
    # zero tokens: arguments checked, nothing enqueued, no device touched
    z = dims(T=0)
    assert L.moe_forward_noalloc(C.byref(z), C.byref(w), None, None, None, None, None,
                                 None) == 0
    assert L.moe_forward_noalloc(C.byref(z), None, None, None, None, None, None, None) == -1


def test_zero_tokens_enqueue_nothing():
    L = lib.load()
    d = dims(T=0)
    w = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000)
    rc = L.moe_forward(C.byref(d), C.byref(w), None, None, None, lib.workspace_bytes(d), None,
                       None, None, None)
    assert rc == 0 and L.moe_last_error().decode() == ""
    rc = L.moe_route(C.byref(d), None, None, None, None, None, None, 0, None)
    assert rc == 0


def test_route_and_plan_refuse_bad_pointers():
    L = lib.load()
    d = dims()
    rc = L.moe_route(C.byref(d), _fake(0x1000), None, None, _fake(0x2000), _fake(0x3000),
                     _fake(0x4000), 1 << 20, None)
    assert rc == -1 and "router_w" in L.moe_last_error().decode()
    rc = L.moe_route(C.byref(d), _fake(0x1004), _fake(0x1000), None, _fake(0x2000),
                     _fake(0x3000), _fake(0x4000), 1 << 20, None)
    assert rc == -3 and "x" in L.moe_last_error().decode()
    rc = L.moe_route(C.byref(d), _fake(0x1000), _fake(0x1000), None, _fake(0x2000),
                     _fake(0x3000), _fake(0x4000), 16, None)
    assert rc == -5 and "workspace_bytes = 16" in L.moe_last_error().decode()
    rc = L.moe_plan(C.byref(d), _fake(0x1000), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                    _fake(0x1000), None, _fake(0x1000), 0, None)
    assert rc == -5


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(lib, "_lib", None)
    monkeypatch.setattr(lib, "LIBPATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        lib.load()


def test_tiles_bytes_and_pack_refusals():
    # the tile-packed copy: E * n_tiles * K * 512 bytes, n_tiles over 128
    # gate columns (SwiGLU up) or 256 rows (relu^2 up, down)
    L = lib.load()
    lfm2 = dims(T=0, H=2048, I=1792, E=32, k=4)
    assert lib.tiles_bytes(lfm2, "up") == 32 * 14 * 2048 * 512 == 32 * 2 * 1792 * 2048 * 2
    assert lib.tiles_bytes(lfm2, "down") == 32 * 8 * 1792 * 512 == 32 * 2048 * 1792 * 2
    relu2 = dims(T=0, H=2688, I=1856, E=128, k=6, act="relu2")
    assert lib.tiles_bytes(relu2, "up") == 128 * 8 * 2688 * 512       # 1856 rows -> 2048
    assert lib.tiles_bytes(relu2, "down") == 128 * 11 * 1856 * 512    # 2688 rows -> 2816
    ragged = dims(T=0, H=128, I=192, E=3, k=2)
    assert lib.tiles_bytes(ragged, "up") == 3 * 2 * 128 * 512         # 192 gate columns -> 256
    # block-FP8 codes: one byte per weight
    fp8 = dims(T=0, H=2048, I=1792, E=32, k=4, wfmt="fp8")
    assert lib.tiles_bytes(fp8, "up") == lib.tiles_bytes(lfm2, "up") // 2
    n = C.c_size_t()
    # bf16 and block-FP8 experts only; which is 0 or 1
    for fmt in ("affine4", "nvfp4", "mxfp4"):
        assert L.moe_tiles_bytes(C.byref(dims(wfmt=fmt, H=256, I=256)), 0, C.byref(n)) == -4
        assert "bf16 and block-FP8" in L.moe_last_error().decode()
    assert L.moe_tiles_bytes(C.byref(lfm2), 2, C.byref(n)) == -4
    assert "which = 2" in L.moe_last_error().decode()
    assert L.moe_tiles_bytes(C.byref(lfm2), 0, None) == -1
    # pack: a short destination, NULL and misaligned pointers, before any launch
    need = lib.tiles_bytes(ragged, "up")
    f = L.moe_pack_tiles
    assert f(C.byref(ragged), 0, _fake(0x1000), _fake(0x2000), need - 1, None) == -5
    assert str(need) in L.moe_last_error().decode()
    assert f(C.byref(ragged), 0, None, _fake(0x2000), need, None) == -1
    assert f(C.byref(ragged), 1, _fake(0x1000), _fake(0x2008), need, None) == -3
    assert "tiles" in L.moe_last_error().decode()


def test_forward_refuses_tiles_of_quantized_experts():
    L = lib.load()
    w = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000, w_up_scales=0x4000,
                    w_down_scales=0x5000, w_up_tiles=0x6000)
    d = dims(wfmt="mxfp4", H=256, I=256)
    rc = L.moe_forward(C.byref(d), C.byref(w), _fake(0x1000), _fake(0x1000), _fake(0x1000),
                       1 << 30, None, None, None, None)
    assert rc == -4 and "w_up_tiles" in L.moe_last_error().decode()
    w = lib.Weights(router_w=0x1000, w_up=0x2000, w_down=0x3000, w_down_tiles=0x6008)
    rc = L.moe_forward(C.byref(dims()), C.byref(w), _fake(0x1000), _fake(0x1000),
                       _fake(0x1000), 1 << 30, None, None, None, None)
    assert rc == -3 and "w_down_tiles" in L.moe_last_error().decode()
