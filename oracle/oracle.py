"""ctypes wrapper of ``oracle.c`` (test infrastructure only).

The C source is the oracle: plain loops, fp32 router in a fixed order,
float64 everywhere after the selection. This file only builds it with gcc
and marshals NumPy arrays; it holds no step of the block's arithmetic.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")
# ORACLE_LIB points the wrapper at another build of oracle.c (the mutation
# tests load deliberately broken copies this way).
LIBPATH = os.environ.get("ORACLE_LIB") or DEFAULT_LIB
CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-Wall", "-Wextra", "-Werror"]

_lib = None
SCORES = {"sigmoid": 0, "softmax": 1}


def compile_source(source: str, out: str, werror: bool = True) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    flags = CFLAGS if werror else [f for f in CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always, unless force is False and it exists)."""
    if force or not os.path.exists(DEFAULT_LIB) or \
            os.path.getmtime(DEFAULT_LIB) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, DEFAULT_LIB)
    return DEFAULT_LIB


class Layer(C.Structure):
    _fields_ = [
        ("T", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
        ("act", C.c_int32), ("wfmt", C.c_int32), ("group", C.c_int32), ("norm_topk", C.c_int32),
        ("I_shared", C.c_int32), ("norm_eps", C.c_double), ("rsf", C.c_double),
        ("x", C.c_void_p), ("router_w", C.c_void_p), ("bias", C.c_void_p),
        ("w_up", C.c_void_p), ("w_up_scales", C.c_void_p), ("w_up_biases", C.c_void_p),
        ("w_down", C.c_void_p), ("w_down_scales", C.c_void_p), ("w_down_biases", C.c_void_p),
        ("shared_up", C.c_void_p), ("shared_down", C.c_void_p),
        ("score_fn", C.c_int32), ("swiglu_limit", C.c_double), ("round_h", C.c_int32),
        ("w_up_global", C.c_void_p), ("w_down_global", C.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if "ORACLE_LIB" not in os.environ and (
                not os.path.exists(LIBPATH) or os.path.getmtime(LIBPATH) < os.path.getmtime(SOURCE)):
            build()
        L = C.CDLL(LIBPATH)
        p = C.c_void_p
        i = C.c_int
        L.oracle_exp32.restype = C.c_float
        L.oracle_exp32.argtypes = [C.c_float]
        L.oracle_sigmoid32.restype = C.c_float
        L.oracle_sigmoid32.argtypes = [C.c_float]
        L.oracle_exp32_many.argtypes = [p, i, p]
        L.oracle_sigmoid32_many.argtypes = [p, i, p]
        L.oracle_topk.argtypes = [p, i, i, p]
        L.oracle_route.argtypes = [i, i, i, i, p, p, p, i, i, C.c_double, p, p, p, p, i]
        L.oracle_softmax32_row.argtypes = [p, i, p]
        L.oracle_add_rmsnorm.argtypes = [i, i, p, p, p, C.c_double, p, p]
        L.oracle_fp8_decode.argtypes = [p, i, p]
        L.oracle_fp4_decode.argtypes = [p, i, p]
        L.oracle_e8m0_decode.argtypes = [p, i, p]
        L.oracle_plan.argtypes = [i, i, i, p, p, p, p, p]
        L.oracle_forward_tokens.argtypes = [C.POINTER(Layer), p, i, p, p, p, i]
        L.oracle_forward_tokens.restype = C.c_int
        L.oracle_affine4_decode.argtypes = [p, p, p, i, i, i, p]
        L.oracle_max_threads.restype = C.c_int
        L.oracle_activate.restype = C.c_double
        L.oracle_activate.argtypes = [i, C.c_double, C.c_double, C.c_double]
        L.oracle_combine32.argtypes = [i, i, i, p, p, p, C.c_float, i, p]
        L.oracle_epilogue32.restype = C.c_uint16
        L.oracle_epilogue32.argtypes = [i, C.c_float, C.c_float]
        L.oracle_expert_rows32.restype = C.c_int
        L.oracle_expert_rows32.argtypes = [C.POINTER(Layer), p, i, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return lib().oracle_max_threads()


def exp32(v) -> np.ndarray:
    v = _c(np.atleast_1d(v), np.float32)
    out = np.empty_like(v)
    lib().oracle_exp32_many(_ptr(v), v.size, _ptr(out))
    return out


def sigmoid32(z) -> np.ndarray:
    z = _c(np.atleast_1d(z), np.float32)
    out = np.empty_like(z)
    lib().oracle_sigmoid32_many(_ptr(z), z.size, _ptr(out))
    return out


def activate(act: str, g: float, u: float, limit: float = 0.0) -> float:
    """The expert activation in float64: act "swiglu" -> silu(g)*u (g capped
    at limit, u clamped to [-limit, limit] when limit > 0), "relu2" -> relu(u)^2."""
    return lib().oracle_activate(0 if act == "swiglu" else 1, float(g), float(u), float(limit))


def softmax32(z) -> np.ndarray:
    """Softmax scores of one router row (fp32 in, fp32 out)."""
    z = _c(np.atleast_1d(z), np.float32)
    out = np.empty_like(z)
    lib().oracle_softmax32_row(_ptr(z), z.size, _ptr(out))
    return out


def topk(keys, k: int) -> np.ndarray:
    keys = _c(keys, np.float32)
    ids = np.empty(k, dtype=np.int32)
    lib().oracle_topk(_ptr(keys), keys.size, k, _ptr(ids))
    return ids


def route(x, router_w, bias, k: int, norm_topk: bool = True, eps: float = 1e-6,
          want_scores: bool = False, nthreads: int = 0, score: str = "sigmoid"):
    """Route every token (score "sigmoid" or "softmax"). Returns ids [T,k]
    int32 and w [T,k] float64, plus z and s [T,E] fp32 when want_scores."""
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = router_w.shape[0]
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    z = np.empty((T, E), dtype=np.float32) if want_scores else None
    s = np.empty((T, E), dtype=np.float32) if want_scores else None
    lib().oracle_route(T, H, E, k, _ptr(x), _ptr(router_w), _ptr(bias), SCORES[score],
                       int(norm_topk), eps, _ptr(z), _ptr(s), _ptr(ids), _ptr(w), nthreads)
    if want_scores:
        return ids, w, z, s
    return ids, w


def plan(ids, E: int):
    """Counting sort of the assignments by expert. Returns counts [E],
    offsets [E+1], sorted [A], slot_of [A] (int32)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    A = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    srt = np.empty(A, dtype=np.int32)
    slot = np.empty(A, dtype=np.int32)
    lib().oracle_plan(T, k, E, _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(srt), _ptr(slot))
    return counts, offsets, srt, slot


def _layer(wl, inp: dict, keep: dict, round_h: bool = False) -> Layer:
    """The oracle_layer struct of a workload's arrays (kept alive in keep)."""
    def arr(name, dtype):
        a = inp.get(name)
        if a is None:
            return None
        a = _c(a, dtype)
        keep[name] = a
        return a.ctypes.data

    affine = wl.wfmt == "affine4"
    fp8 = wl.wfmt == "fp8"
    fp4 = wl.wfmt in ("nvfp4", "mxfp4")
    code_t = np.uint32 if affine else np.uint8 if (fp8 or fp4) else np.uint16
    scale_t = np.float32 if fp8 else np.uint8 if fp4 else np.uint16
    return Layer(T=wl.T, H=wl.H, I=wl.I, E=wl.E, k=wl.k,
                 act=0 if wl.act == "swiglu" else 1,
                 wfmt={"bf16": 0, "affine4": 1, "fp8": 2, "nvfp4": 3, "mxfp4": 4}[wl.wfmt],
                 group=wl.group if affine else 0, norm_topk=int(wl.norm_topk),
                 I_shared=wl.I_shared, norm_eps=wl.norm_eps, rsf=wl.rsf,
                 x=arr("x", np.uint16), router_w=arr("router_w", np.float32),
                 bias=arr("bias", np.float32),
                 w_up=arr("w_up", code_t),
                 w_up_scales=arr("w_up_scales", scale_t),
                 w_up_biases=arr("w_up_biases", np.uint16),
                 w_down=arr("w_down", code_t),
                 w_down_scales=arr("w_down_scales", scale_t),
                 w_down_biases=arr("w_down_biases", np.uint16),
                 shared_up=arr("shared_up", np.uint16) if wl.I_shared else None,
                 shared_down=arr("shared_down", np.uint16) if wl.I_shared else None,
                 score_fn=SCORES[getattr(wl, "score", "sigmoid")],
                 swiglu_limit=float(getattr(wl, "swiglu_limit", 0.0)),
                 round_h=int(round_h),
                 w_up_global=arr("w_up_global", np.float32),
                 w_down_global=arr("w_down_global", np.float32))


def forward_tokens(wl, inp: dict, tokens, nthreads: int = 0, want_routing: bool = False,
                   round_h: bool = False):
    """The block's float64 output rows for ``tokens`` ([n, H] float64).

    ``wl`` carries the shapes and flags (a workloads.Workload or anything
    with the same attributes); ``inp`` the arrays from workloads.generate.
    round_h: the activation between the projections rounded to bf16, as the
    path stores it (everything else stays float64).
    """
    tokens = _c(np.atleast_1d(tokens), np.int32)
    keep = {}
    L = _layer(wl, inp, keep, round_h)
    n = tokens.size
    out = np.empty((n, wl.H), dtype=np.float64)
    ids = np.empty((n, wl.k), dtype=np.int32)
    w = np.empty((n, wl.k), dtype=np.float64)
    rc = lib().oracle_forward_tokens(C.byref(L), _ptr(tokens), n, _ptr(out), _ptr(ids), _ptr(w),
                                     nthreads)
    if rc != 0:
        raise ValueError("token index out of range")
    if want_routing:
        return out, ids, w
    return out


def combine32(w, y, shared, rsf: float, fold: bool = False) -> np.ndarray:
    """fp32 mimic of the engine's combine, for bitwise pins: w [n,k] fp32,
    y [n,k,H] fp32, shared [n,H] fp32 or None. out = (fma chain of w_j y_j,
    j ascending) * rsf + shared; fold=True gives the folded form
    (fma chain of (rsf w_j) y_j) + shared instead."""
    w = _c(w, np.float32)
    y = _c(y, np.float32)
    shared = _c(shared, np.float32)
    n, k, H = y.shape
    assert w.shape == (n, k)
    out = np.empty((n, H), dtype=np.float32)
    lib().oracle_combine32(n, H, k, _ptr(w), _ptr(y), _ptr(shared), C.c_float(rsf), int(fold),
                           _ptr(out))
    return out


def epilogue32(act: str, g, u) -> np.ndarray:
    """fp32 epilogue rounded once to bf16 (bits): relu^2 of u, or
    (g * sigmoid32(g)) * u for SwiGLU."""
    g = np.broadcast_to(np.asarray(g, np.float32), np.shape(u)).ravel()
    u = np.asarray(u, np.float32).ravel()
    a = 0 if act == "swiglu" else 1
    f = lib().oracle_epilogue32
    return np.array([f(a, C.c_float(gi), C.c_float(ui)) for gi, ui in zip(g, u)], dtype=np.uint16)


def expert_rows32(wl, inp: dict, tokens, ids):
    """Per-assignment fp32 down rows y [n,k,H] and the shared expert's fp32
    output [n,H] (or None) for ``tokens`` routed to ``ids`` [n,k], with the
    fp32 epilogue rounded once to bf16 between the projections. Returns
    (y, shared, inexact): inexact counts projection values that were not
    exact in fp32 (0 on data with one non-zero term per dot product)."""
    tokens = _c(np.atleast_1d(tokens), np.int32)
    ids = _c(ids, np.int32)
    keep = {}
    L = _layer(wl, inp, keep)
    n = tokens.size
    assert ids.shape == (n, wl.k)
    y = np.empty((n, wl.k, wl.H), dtype=np.float32)
    sh = np.empty((n, wl.H), dtype=np.float32) if wl.I_shared else None
    inexact = lib().oracle_expert_rows32(C.byref(L), _ptr(tokens), n, _ptr(ids), _ptr(y), _ptr(sh))
    return y, sh, inexact


def affine4_decode(codes, scales, biases, group: int = 64) -> np.ndarray:
    """Dequantise affine-4 rows exactly: codes [rows, K/8] uint32, scales and
    biases [rows, K/group] bf16 bits -> [rows, K] float64."""
    codes = _c(codes, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    rows, kw = codes.shape
    K = kw * 8
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_affine4_decode(_ptr(codes), _ptr(scales), _ptr(biases), rows, K, group, _ptr(out))
    return out


def add_rmsnorm(h, residual, gamma, eps: float = 1e-5):
    """Fused residual add + RMSNorm: h (or None) and residual bf16 bits
    [T,H], gamma bf16 bits [H]. Returns the new residual (bf16 bits, [T,H])
    and x in float64 ([T,H])."""
    residual = _c(residual, np.uint16)
    h = _c(h, np.uint16)
    gamma = _c(gamma, np.uint16)
    T, H = residual.shape
    res_out = np.empty((T, H), dtype=np.uint16)
    x = np.empty((T, H), dtype=np.float64)
    lib().oracle_add_rmsnorm(T, H, _ptr(h), _ptr(residual), _ptr(gamma), eps, _ptr(res_out),
                             _ptr(x))
    return res_out, x


def fp8_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, exactly."""
    codes = _c(np.atleast_1d(codes), np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib().oracle_fp8_decode(_ptr(codes), codes.size, _ptr(out))
    return out


def fp4_decode(packed, n: int) -> np.ndarray:
    """The first n FP4 E2M1 values of a packed byte array (element c in byte
    c // 2, low nibble first), as float64."""
    packed = _c(np.asarray(packed).reshape(-1), np.uint8)
    assert 0 <= n <= 2 * packed.size
    out = np.empty(n, dtype=np.float64)
    lib().oracle_fp4_decode(_ptr(packed), n, _ptr(out))
    return out


def e8m0_decode(codes) -> np.ndarray:
    """OCP MX E8M0 scale bytes -> float64: 2^(b - 127), 0xFF NaN."""
    codes = _c(np.atleast_1d(codes), np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib().oracle_e8m0_decode(_ptr(codes), codes.size, _ptr(out))
    return out
