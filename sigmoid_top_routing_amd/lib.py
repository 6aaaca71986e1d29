"""Python binding of libmoe (include/moe.h) over ctypes.

Argument marshalling only: tensors are torch tensors on the GPU, passed by
data pointer together with torch's current HIP stream; every step of the
block runs in the library's HIP kernels. If libmoe.so has not been built,
loading fails with an error; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_E_NULL", -2: "MOE_E_SHAPE", -3: "MOE_E_ALIGN",
          -4: "MOE_E_UNSUPPORTED", -5: "MOE_E_WORKSPACE", -6: "MOE_E_HIP"}
ACT = {"swiglu": 0, "relu2": 1}
WFMT = {"bf16": 0, "affine4": 1, "fp8": 2, "nvfp4": 3, "mxfp4": 4}
OUT = {torch.bfloat16: 0, torch.float32: 1}
SCORE = {"sigmoid": 0, "softmax": 1}

# every entry point include/moe.h declares
EXPORTS = ("moe_workspace_bytes", "moe_tiles_bytes", "moe_pack_tiles", "moe_route", "moe_plan",
           "moe_forward", "moe_forward_profiled", "moe_forward_noalloc", "moe_add_rmsnorm",
           "moe_last_error")
TILES = {"up": 0, "down": 1}
NOALLOC_SCRATCH_BYTES = 64 << 20
PROFILE_EVENTS = 7
STAGES = ("route", "plan", "up", "down", "shared", "combine")


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Dims(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32),
                ("k", C.c_int32), ("act", C.c_int32), ("wfmt", C.c_int32), ("group", C.c_int32),
                ("norm_topk", C.c_int32), ("norm_eps", C.c_float), ("routed_scale", C.c_float),
                ("I_shared", C.c_int32), ("out_dtype", C.c_int32), ("score_fn", C.c_int32),
                ("swiglu_limit", C.c_float), ("fold_routed_scale", C.c_int32),
                ("row_invariant", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "router_w", "expert_bias", "w_up", "w_up_scales", "w_up_biases", "w_down",
        "w_down_scales", "w_down_biases", "shared_up", "shared_down", "w_up_global",
        "w_down_global", "w_up_tiles", "w_down_tiles")]


_lib = None


def load():
    """Load libmoe.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise RuntimeError(f"{LIBPATH} is not built: run `python -m sigmoid_top_routing_amd.build`")
        L = C.CDLL(LIBPATH)
        p, i = C.c_void_p, C.c_int
        L.moe_workspace_bytes.argtypes = [C.POINTER(Dims), C.POINTER(C.c_size_t)]
        L.moe_workspace_bytes.restype = i
        L.moe_tiles_bytes.argtypes = [C.POINTER(Dims), C.c_int32, C.POINTER(C.c_size_t)]
        L.moe_tiles_bytes.restype = i
        L.moe_pack_tiles.argtypes = [C.POINTER(Dims), C.c_int32, p, p, C.c_size_t, p]
        L.moe_pack_tiles.restype = i
        L.moe_route.argtypes = [C.POINTER(Dims), p, p, p, p, p, p, C.c_size_t, p]
        L.moe_route.restype = i
        L.moe_plan.argtypes = [C.POINTER(Dims), p, p, p, p, p, p, p, C.c_size_t, p]
        L.moe_plan.restype = i
        L.moe_forward.argtypes = [C.POINTER(Dims), C.POINTER(Weights), p, p, p, C.c_size_t, p,
                                  p, p, p]
        L.moe_forward.restype = i
        L.moe_forward_profiled.argtypes = [C.POINTER(Dims), C.POINTER(Weights), p, p, p,
                                           C.c_size_t, p, p, p, p, C.POINTER(p)]
        L.moe_forward_profiled.restype = i
        L.moe_forward_noalloc.argtypes = [C.POINTER(Dims), C.POINTER(Weights), p, p, p, p, p,
                                          p]
        L.moe_forward_noalloc.restype = i
        L.moe_add_rmsnorm.argtypes = [C.c_int32, C.c_int32, p, p, p, C.c_float, p, p, p]
        L.moe_add_rmsnorm.restype = i
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, load().moe_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_dims(T, H, I, E, k, act="swiglu", wfmt="bf16", rsf=1.0, I_shared=0, norm_topk=True,
              norm_eps=1e-6, out_dtype=torch.bfloat16, score="sigmoid",
              swiglu_limit=0.0, fold_routed_scale=False, row_invariant=False) -> Dims:
    return Dims(T=T, H=H, I=I, E=E, k=k, act=ACT[act], wfmt=WFMT[wfmt],
                group=64 if wfmt == "affine4" else 0, norm_topk=int(norm_topk),
                norm_eps=norm_eps, routed_scale=rsf, I_shared=I_shared, out_dtype=OUT[out_dtype],
                score_fn=SCORE[score], swiglu_limit=swiglu_limit,
                fold_routed_scale=int(fold_routed_scale), row_invariant=int(row_invariant))


def workspace_bytes(d: Dims) -> int:
    n = C.c_size_t()
    _check(load().moe_workspace_bytes(C.byref(d), C.byref(n)))
    return n.value


def tiles_bytes(d: Dims, which: str) -> int:
    """Bytes of the tile-packed copy of w_up ("up") or w_down ("down") (moe_tiles_bytes)."""
    n = C.c_size_t()
    _check(load().moe_tiles_bytes(C.byref(d), TILES[which], C.byref(n)))
    return n.value


def pack_tiles(d: Dims, which: str, w, stream=None) -> torch.Tensor:
    """The tile-packed copy of a bf16 or FP8 weight tensor (moe_pack_tiles),
    as a flat uint8 tensor on w's device."""
    n = tiles_bytes(d, which)
    tiles = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check(load().moe_pack_tiles(C.byref(d), TILES[which], _ptr(w), _ptr(tiles), n,
                                 _stream(stream)))
    return tiles


def route(x, router_w, bias, k, norm_topk=True, norm_eps=1e-6, stream=None, score="sigmoid"):
    """ids [T,k] int32 and weights [T,k] fp32 (moe_route)."""
    T, H = x.shape
    E = router_w.shape[0]
    d = make_dims(T, H, 64, E, k, norm_topk=norm_topk, norm_eps=norm_eps, score=score)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    nbytes = workspace_bytes(d)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(load().moe_route(C.byref(d), _ptr(x), _ptr(router_w), _ptr(bias), _ptr(ids), _ptr(w),
                            _ptr(ws), nbytes, _stream(stream)))
    return ids, w


def add_rmsnorm(residual, gamma, eps=1e-5, h=None, residual_out=None, x=None, stream=None):
    """Fused residual add + RMSNorm (moe_add_rmsnorm): bf16 [T,H] residual and
    optional h, bf16 [H] gamma. Returns (residual_out, x); pass
    residual_out=residual to update the residual in place."""
    T, H = residual.shape
    if residual_out is None and h is not None:
        residual_out = torch.empty_like(residual)
    if x is None:
        x = torch.empty_like(residual)
    _check(load().moe_add_rmsnorm(T, H, _ptr(h), _ptr(residual), _ptr(gamma), eps,
                                  _ptr(residual_out), _ptr(x), _stream(stream)))
    return residual_out, x


def plan(ids, E, fault=None, stream=None):
    """counts [E], offsets [E+1], sorted [T*k], slot_of [T*k] (moe_plan)."""
    T, k = ids.shape
    d = make_dims(T, 64, 64, E, k)
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    nbytes = workspace_bytes(d)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(load().moe_plan(C.byref(d), _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(srt),
                           _ptr(slot), _ptr(fault), _ptr(ws), nbytes, _stream(stream)))
    return counts, offsets, srt, slot


@dataclass
class MoEBlock:
    """One MoE layer's weights on the device and its options.

    Weight tensors follow include/moe.h: router_w fp32 [E,H], bias fp32 [E]
    or None, w_up / w_down bf16 (or uint32 codes with bf16 scales and
    biases for "affine4"), shared_up / shared_down bf16 or None.
    """
    H: int
    I: int
    E: int
    k: int
    router_w: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    bias: torch.Tensor | None = None
    w_up_scales: torch.Tensor | None = None
    w_up_biases: torch.Tensor | None = None
    w_down_scales: torch.Tensor | None = None
    w_down_biases: torch.Tensor | None = None
    w_up_global: torch.Tensor | None = None      # NVFP4: fp32 [E]
    w_down_global: torch.Tensor | None = None
    shared_up: torch.Tensor | None = None
    shared_down: torch.Tensor | None = None
    w_up_tiles: torch.Tensor | None = None       # tile-packed copies (pack_tiles)
    w_down_tiles: torch.Tensor | None = None
    act: str = "swiglu"
    wfmt: str = "bf16"
    rsf: float = 1.0
    I_shared: int = 0
    norm_topk: bool = True
    norm_eps: float = 1e-6
    score: str = "sigmoid"
    swiglu_limit: float = 0.0
    fold_routed_scale: bool = False
    row_invariant: bool = False

    def __post_init__(self):
        self._ws = None
        self._calls = {}     # per-call marshalling, keyed by everything it depends on

    def _options(self):
        return (self.H, self.I, self.E, self.k, self.act, self.wfmt, self.rsf, self.I_shared,
                self.norm_topk, self.norm_eps, self.score, self.swiglu_limit,
                self.fold_routed_scale, self.row_invariant)

    def dims(self, T, out_dtype=torch.bfloat16) -> Dims:
        return make_dims(T, self.H, self.I, self.E, self.k, self.act, self.wfmt, self.rsf,
                         self.I_shared, self.norm_topk, self.norm_eps, out_dtype, self.score,
                         self.swiglu_limit, self.fold_routed_scale, self.row_invariant)

    def _weight_ptrs(self):
        return (_ptr(self.router_w), _ptr(self.bias), _ptr(self.w_up), _ptr(self.w_up_scales),
                _ptr(self.w_up_biases), _ptr(self.w_down), _ptr(self.w_down_scales),
                _ptr(self.w_down_biases), _ptr(self.shared_up), _ptr(self.shared_down),
                _ptr(self.w_up_global), _ptr(self.w_down_global), _ptr(self.w_up_tiles),
                _ptr(self.w_down_tiles))

    def weights(self) -> Weights:
        (rw, b, wu, wus, wub, wd, wds, wdb, su, sd, ug, dg, ut, dt) = self._weight_ptrs()
        return Weights(router_w=rw, expert_bias=b, w_up=wu, w_up_scales=wus, w_up_biases=wub,
                       w_down=wd, w_down_scales=wds, w_down_biases=wdb, shared_up=su,
                       shared_down=sd, w_up_global=ug, w_down_global=dg, w_up_tiles=ut,
                       w_down_tiles=dt)

    def pack_tiles(self, stream=None):
        """Give the block tile-packed copies of its bf16 or block-FP8 expert
        weights (moe_pack_tiles), which the prompt-sized MFMA tiles then read."""
        d = self.dims(0)
        self.w_up_tiles = pack_tiles(d, "up", self.w_up, stream)
        self.w_down_tiles = pack_tiles(d, "down", self.w_down, stream)
        return self

    def _marshalled(self, T, out_dtype):
        """(dims, weights, workspace bytes) of a call: built once per shape,
        options and weight tensors, so a decode loop does not rebuild them."""
        key = (T, out_dtype, self._options(), self._weight_ptrs())
        hit = self._calls.get(key)
        if hit is None:
            d = self.dims(T, out_dtype)
            hit = (d, self.weights(), workspace_bytes(d))
            if len(self._calls) > 64:
                self._calls.clear()
            self._calls[key] = hit
        return hit

    def workspace(self, d: Dims, device, n=None) -> torch.Tensor:
        n = workspace_bytes(d) if n is None else n
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        return self._ws

    def forward(self, x, out_dtype=torch.bfloat16, out=None, ids_out=None, weights_out=None,
                offsets_out=None, workspace=None, stream=None, events=None):
        """out [T,H] (moe_forward). x is bf16 [T,H] on the GPU.

        events: optional StageEvents; the call then goes through
        moe_forward_profiled and records the stage boundaries on the stream."""
        T = x.shape[0]
        d, w, need = self._marshalled(T, out_dtype)
        if out is None:
            out = torch.empty((T, self.H), dtype=out_dtype, device=x.device)
        ws = workspace if workspace is not None else self.workspace(d, x.device, need)
        args = (C.byref(d), C.byref(w), _ptr(x), _ptr(out), _ptr(ws), ws.numel(), _stream(stream),
                _ptr(ids_out), _ptr(weights_out), _ptr(offsets_out))
        if events is None:
            _check(load().moe_forward(*args))
        else:
            _check(load().moe_forward_profiled(*args, events.handles()))
        return out


    def forward_noalloc(self, x, out_dtype=torch.bfloat16, out=None, ids_out=None,
                        weights_out=None, offsets_out=None, stream=None):
        """out [T,H] through moe_forward_noalloc: the library's static scratch
        instead of a workspace (no allocation inside the call)."""
        T = x.shape[0]
        d = self.dims(T, out_dtype)
        if out is None:
            out = torch.empty((T, self.H), dtype=out_dtype, device=x.device)
        w = self.weights()
        _check(load().moe_forward_noalloc(C.byref(d), C.byref(w), _ptr(x), _ptr(out),
                                          _stream(stream), _ptr(ids_out), _ptr(weights_out),
                                          _ptr(offsets_out)))
        return out


class StageEvents:
    """Seven timing events for moe_forward_profiled (torch.cuda.Event; the
    library records them on the call's stream)."""

    def __init__(self):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(PROFILE_EVENTS)]
        for e in self.ev:
            e.record()           # creates the underlying hipEvent_t
        self._arr = (C.c_void_p * PROFILE_EVENTS)(*[e.cuda_event for e in self.ev])

    def handles(self):
        return self._arr

    def stage_ms(self) -> dict:
        """Milliseconds between consecutive boundaries (call after a sync)."""
        return {name: self.ev[i].elapsed_time(self.ev[i + 1]) for i, name in enumerate(STAGES)}

    def total_ms(self) -> float:
        return self.ev[0].elapsed_time(self.ev[-1])


def block_from_arrays(wl, inp: dict, device="cuda") -> MoEBlock:
    """Upload a workload's NumPy arrays (see workloads.generate) as a MoEBlock."""
    def dev(name, as_bf16=False):
        a = inp.get(name)
        if a is None:
            return None
        t = torch.from_numpy(a.view(a.dtype.str.replace("u", "i")) if a.dtype.kind == "u" else a)
        t = t.to(device)
        return t.view(torch.bfloat16) if as_bf16 else t
    aff = wl.wfmt == "affine4"
    fp8 = wl.wfmt == "fp8"
    nv4 = wl.wfmt == "nvfp4"
    quant = aff or fp8 or nv4 or wl.wfmt == "mxfp4"
    return MoEBlock(H=wl.H, I=wl.I, E=wl.E, k=wl.k, router_w=dev("router_w"), bias=dev("bias"),
                    w_up=dev("w_up", not quant), w_down=dev("w_down", not quant),
                    w_up_scales=dev("w_up_scales", aff),
                    w_up_biases=dev("w_up_biases", True),
                    w_down_scales=dev("w_down_scales", aff),
                    w_down_biases=dev("w_down_biases", True),
                    w_up_global=dev("w_up_global"), w_down_global=dev("w_down_global"),
                    shared_up=dev("shared_up", True), shared_down=dev("shared_down", True),
                    act=wl.act, wfmt=wl.wfmt, rsf=wl.rsf, I_shared=wl.I_shared,
                    norm_topk=wl.norm_topk, norm_eps=wl.norm_eps, score=wl.score,
                    swiglu_limit=wl.swiglu_limit)


def x_to_device(x_bits, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16 NumPy) -> torch bf16 on the device."""
    return torch.from_numpy(x_bits.view("i2")).to(device).view(torch.bfloat16)
