"""Benchmark of the sigmoid top-k routed MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step is one moe_forward over one batch of synthetic input: router,
top-k, plan, grouped expert GEMMs with the fused activation, the shared
expert when the workload has one, and the weighted combine. The default
workload is the LFM2-MoE-shaped prefill chunk (T=4096, H=2048, I=1792,
E=32, top-4, bf16 SwiGLU experts). Inputs are resident in HBM before the
timed region, and the untimed warm-up steps (100 by default) run first
because the part's clock ramps up over about 50 ms of load after idle; each
other configuration gets 50 ms of untimed calls for the same reason. Prints
one JSON line.

bf16 and block-FP8 expert weights get their tile-packed copy (moe_pack_tiles)
once, before any timed call, as a caller does when it loads the weights: the
prompt-sized MFMA tiles read it (the same output bits, each K-slice of a tile
one contiguous 16 KB, 8 KB for FP8); the time of that one-off copy is
reported as pack_tiles_ms. With --no-tiles the tiles read the weights as
stored.

Besides the whole-block throughput the line carries:
  roofline      the dominant kernel (the routed up-projection GEMM) against
                the bf16 MFMA peak (or HBM for a decode-sized batch), timed
                with the library's stage events on the call's stream;
  cpu_baseline  the float64 CPU oracle on a sample of the same tokens;
  decode        the T=8 decode step on the same weights (HBM-bound), with
                the 256 MB last-level cache flushed (by reading 512 MB)
                before every call;
  add_rmsnorm   the fused residual add + RMSNorm that makes the block's input;
  configs       the other workloads, each with its step time, algorithmic
                bytes and flops and their fractions of the HBM and bf16 MFMA
                peaks: the tiny block, the relu^2 block with a shared expert,
                the 4-bit block, the 4-bit decode step (T = 8) without
                and with the four boosted experts, the block-FP8, NVFP4 and
                MXFP4 prefill and decode steps, and the bf16 decode step with
                row_invariant (every batch on the MFMA tiles).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = ("MoE-block tokens/s at 1 MI355X; % bf16 MFMA peak (prefill), % HBM BW (decode)")


def flops_of(wl):
    """Algorithmic MFMA flops of one block call: per assignment 2*n_up*H for
    the up projection and 2*H*I for the down projection, plus the shared
    expert on every token."""
    A = wl.T * wl.k
    up = 2.0 * A * wl.n_up * wl.H
    down = 2.0 * A * wl.H * wl.I
    shared = 0.0
    if wl.I_shared:
        n_sup = 2 * wl.I_shared if wl.act == "swiglu" else wl.I_shared
        shared = 2.0 * wl.T * (n_sup + wl.I_shared) * wl.H
    return up, down, shared


def expert_bytes(wl):
    """Bytes of one expert's (up, down) weights as stored."""
    if wl.wfmt == "affine4":
        up = wl.n_up * wl.H // 2 + 2 * 2 * wl.n_up * (wl.H // 64)
        down = wl.H * wl.I // 2 + 2 * 2 * wl.H * (wl.I // 64)
    elif wl.wfmt == "fp8":
        up = wl.n_up * wl.H + 4 * (wl.n_up // 128) * (wl.H // 128)
        down = wl.H * wl.I + 4 * (wl.H // 128) * (wl.I // 128)
    elif wl.wfmt == "nvfp4":        # codes, an e4m3 scale per 16, the global scale
        up = wl.n_up * wl.H // 2 + wl.n_up * wl.H // 16 + 4
        down = wl.H * wl.I // 2 + wl.H * wl.I // 16 + 4
    elif wl.wfmt == "mxfp4":        # codes, an e8m0 scale per 32
        up = wl.n_up * wl.H // 2 + wl.n_up * wl.H // 32
        down = wl.H * wl.I // 2 + wl.H * wl.I // 32
    else:
        up = 2 * wl.n_up * wl.H
        down = 2 * wl.H * wl.I
    return up, down


def load_traffic(tag, workload, sources):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel sources as they are now; else None."""
    from sigmoid_top_routing_amd import profiling
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{tag}@{workload}")
    if not rec or rec.get("source_digest") != profiling.source_digest(*sources):
        return None
    return rec.get("bytes_per_launch")


# the sources of the kernel the roofline is taken on (bf16 expert GEMMs)
GEMM_SOURCES = ("grouped_gemm.hip", "device.hpp", "kernels.hpp")
COPY_BYTES = 256 << 20


def profile_run(args):
    """Untimed calls for a profiler to wrap: `steps` forward calls of the
    workload, then two copies of COPY_BYTES bytes that scale the HBM byte
    counters: the runtime's device-to-device copy, and an elementwise copy
    (x * 1 in fp32, 16-byte loads and stores like the library's kernels)."""
    import torch
    from sigmoid_top_routing_amd import lib
    from sigmoid_top_routing_amd import workloads as W
    wl = W.by_name(args.workload)
    inp = W.generate(wl)
    block = lib.block_from_arrays(wl, inp)
    if wl.wfmt in ("bf16", "fp8") and not args.no_tiles:
        block.pack_tiles()
    x = lib.x_to_device(inp["x"])
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.steps):
        block.forward(x, out=out)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.mul(src.view(torch.float32), 1.0, out=dst.view(torch.float32))
    torch.cuda.synchronize()
    print(f"profile run: {args.steps} calls of {wl.name}, copy of {COPY_BYTES} bytes", flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, budget_s=15.0):
    """The float64 oracle on a sample of the workload's tokens, on every
    thread OpenMP gives it (the host cores this process may run on), plus
    the whole tiny workload on one thread."""
    import oracle
    from sigmoid_top_routing_amd import workloads as W
    threads = oracle.max_threads()
    rng = np.random.default_rng(1234)
    n0 = max(threads, 4)
    toks = rng.choice(wl.T, size=min(n0, wl.T), replace=False).astype(np.int32)
    t0 = time.perf_counter()
    oracle.forward_tokens(wl, inp, toks)
    dt = time.perf_counter() - t0
    n = int(min(wl.T, max(n0, n0 * budget_s / max(dt, 1e-3))))
    toks = rng.choice(wl.T, size=n, replace=False).astype(np.int32)
    t0 = time.perf_counter()
    oracle.forward_tokens(wl, inp, toks)
    dt = time.perf_counter() - t0
    tiny = W.TINY
    tin = W.generate(tiny)
    t1 = time.perf_counter()
    oracle.forward_tokens(tiny, tin, np.arange(tiny.T), nthreads=1)
    dt1 = time.perf_counter() - t1
    oracle.forward_tokens(tiny, tin, np.arange(1), nthreads=threads)   # restores the count
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of the {wl.T} tokens of {wl.name} (routing and float64 experts "
                      f"per token), {dt:.1f} s on {threads} threads",
            "host_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "tiny_one_thread": {"workload": tiny.name, "tokens": tiny.T, "s": dt1,
                                "tokens_per_s": tiny.T / dt1}}


def variant(wl, args):
    """The workload with the router scores or SwiGLU limit the flags ask for
    (its name then says so)."""
    kw = {}
    if args.score is not None and args.score != wl.score:
        kw["score"] = args.score
    if args.swiglu_limit is not None and args.swiglu_limit != wl.swiglu_limit:
        kw["swiglu_limit"] = args.swiglu_limit
    if not kw:
        return wl
    tag = "".join(f"+{k}={v}" for k, v in kw.items())
    return wl.with_(name=wl.name + tag, **kw)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the part's clock ramps up over the first ~50 ms of load after idle (the
    # LFM2 prefill step runs 614 us in its first 10 calls, 500 us from about
    # the 60th on): 100 untimed steps put the timed region at steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="lfm2_prefill_t4096")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--score", choices=("sigmoid", "softmax"), default=None,
                    help="router scores in place of the workload's own")
    ap.add_argument("--swiglu-limit", type=float, default=None,
                    help="SwiGLU input limit in place of the workload's own")
    ap.add_argument("--no-tiles", action="store_true",
                    help="no tile-packed copy of the bf16 expert weights")
    ap.add_argument("--profile-run", action="store_true",
                    help="untimed calls plus a calibration copy, for rocprofv3 to wrap")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} asked for)", file=sys.stderr)
        sys.exit(2)
    if args.profile_run:
        profile_run(args)
        return

    import torch
    from sigmoid_top_routing_amd import lib
    from sigmoid_top_routing_amd import workloads as W

    wl = variant(W.by_name(args.workload), args)
    inp = W.generate(wl)
    block = lib.block_from_arrays(wl, inp)
    tiles = wl.wfmt in ("bf16", "fp8") and not args.no_tiles
    pack_ms = pack(block, torch) if tiles else None
    x = lib.x_to_device(inp["x"])
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    block.workspace(block.dims(wl.T), x.device)

    for _ in range(args.warmup):
        block.forward(x, out=out, ids_out=ids)
    # timed region 1: plain calls, the block's throughput
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        block.forward(x, out=out, ids_out=ids)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    # timed region 2: the same calls with stage events recorded on the call's
    # stream (each record costs a few microseconds of queue time, so the
    # throughput above is taken without them)
    evs = [lib.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        block.forward(x, out=out, ids_out=ids, events=evs[i])
    torch.cuda.synchronize()
    stages = {k: float(np.mean([e.stage_ms()[k] for e in evs])) for k in lib.STAGES}

    up_f, down_f, sh_f = flops_of(wl)
    total_f = up_f + down_f + sh_f
    ids_np = ids.cpu().numpy()
    D = int(np.unique(ids_np).size)
    eb_up, eb_down = expert_bytes(wl)
    A = wl.T * wl.k
    decode_sized = A <= 64
    if decode_sized:
        algo = D * eb_up + wl.T * wl.H * 2 + A * wl.I * 2
        achieved = algo / (stages["up"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "routed up-projection GEMM", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = up_f / (stages["up"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "routed up-projection GEMM", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    roof["traffic"] = load_traffic("gemm_up", wl.name, GEMM_SOURCES)
    roof["avg_launch_us"] = 1e3 * stages["up"]
    # which calls the launch time comes from (not the throughput region's,
    # which records no events; the kernel trace of the same command gives the
    # same calls' dispatch times, a few microseconds below these)
    roof["timing"] = ("HIP events on the call's stream around the up stage, mean of the %d calls "
                      "with stage events that follow the timed region" % args.steps)

    result = {
        "metric": METRIC,
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
                   "act": wl.act, "weights": wl.wfmt, "rsf": wl.rsf, "I_shared": wl.I_shared,
                   "score": wl.score, "swiglu_limit": wl.swiglu_limit,
                   "tile_packed_weights": tiles, "parallelism": "single GPU"},
        "pack_tiles_ms": pack_ms,
        "roofline": roof,
        "block": {"tflops": total_f / (ms_per_step * 1e-3) / 1e12,
                  "frac_bf16_peak": total_f / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "distinct_experts": D, "stages_ms": stages},
    }

    if not args.no_decode and wl.name.startswith("lfm2_prefill_t4096"):
        print("bench: decode, add + RMSNorm and the other configurations", file=sys.stderr,
              flush=True)
        result["decode"] = bench_step(W.DECODE, W, lib, torch, block=block, flush=True)
        result["add_rmsnorm"] = bench_norm(wl.T, wl.H, W, lib, torch)
        result["configs"] = {}
        for tag, name, flush in (("tiny", "tiny_t64_e8_k2", False),
                                 ("relu2", "nemotron_relu2_t2048", False),
                                 ("affine4", "affine4_t1024", False),
                                 ("affine4_decode", "affine4_flat_decode_t8", True),
                                 ("affine4_decode_boosted", "affine4_decode_t8", True),
                                 ("fp8", "lfm2_fp8_prefill_t4096", False),
                                 ("fp8_decode", "lfm2_fp8_decode_t8", True),
                                 ("nvfp4", "lfm2_nvfp4_prefill_t4096", False),
                                 ("nvfp4_decode", "lfm2_nvfp4_decode_t8", True),
                                 ("mxfp4", "lfm2_mxfp4_prefill_t4096", False),
                                 ("mxfp4_decode", "lfm2_mxfp4_decode_t8", True)):
            result["configs"][tag] = bench_step(W.by_name(name), W, lib, torch, flush=flush,
                                                tiles=not args.no_tiles)
            print(f"bench: {tag} done", file=sys.stderr, flush=True)
        result["configs"]["decode_row_invariant"] = bench_step(W.DECODE, W, lib, torch, block=block,
                                                               flush=True, row_invariant=True)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(result))


def bench_norm(T, H, W, lib, torch, steps=20):
    """The fused residual add + RMSNorm that makes the block's input, on the
    block's shape: one event pair around each call on the current stream,
    each call after a 512 MB read that evicts the last-level cache (its 67 MB
    would otherwise stay there between calls); the median call is reported.
    Algorithmic bytes: h and residual read, residual and x written (bf16),
    plus gamma."""
    d = W.norm_inputs(T, H, seed=1)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).to("cuda")
    h, res, g = dev(d["h"]), dev(d["residual"]), dev(d["gamma"])
    res_out, x = torch.empty_like(res), torch.empty_like(res)
    flush = torch.ones(64 << 20, dtype=torch.int64, device="cuda")
    warm(torch, lambda: lib.add_rmsnorm(res, g, d["eps"], h=h, residual_out=res_out, x=x))
    times = []
    for _ in range(steps):
        flush.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        lib.add_rmsnorm(res, g, d["eps"], h=h, residual_out=res_out, x=x)
        b.record()
        torch.cuda.synchronize()
        times.append(1e3 * a.elapsed_time(b))
    us = float(np.median(times))
    algo = 4 * T * H * 2 + H * 2
    gbs = algo / (us * 1e-6) / 1e9
    return {"T": T, "H": H, "us_per_call": us, "algorithmic_bytes": algo, "GBps": gbs,
            "frac_hbm": gbs / PEAK_HBM_GBS, "timing": "median of %d calls, cache evicted" % steps}


def pack(block, torch):
    """The block's tile-packed weight copies (moe_pack_tiles), made once;
    returns the milliseconds the copy took on the GPU."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    block.pack_tiles()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def warm(torch, fn, ms=50.0):
    """Untimed calls of fn until `ms` milliseconds of them have run (at least
    three): the clock ramps up over about 50 ms of load after idle, and the
    host work between configurations (input generation, uploads) idles it."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or 1e3 * (time.perf_counter() - t0) < ms:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        n += 5


def shared_bytes(wl):
    if not wl.I_shared:
        return 0
    n_sup = 2 * wl.I_shared if wl.act == "swiglu" else wl.I_shared
    return 2 * (n_sup + wl.I_shared) * wl.H


def bench_step(wl, W, lib, torch, block=None, flush=False, steps=20, row_invariant=False,
               tiles=True):
    """One workload's step, each call between its own event pair on the
    current stream (the median call is reported), then the stage breakdown
    from calls with the stage events inside (each record adds a few
    microseconds of queue time, so the step time is taken without them).
    flush: before every call a 512 MB buffer is read (twice the 256 MB
    last-level cache) so the expert weights come from HBM; it is read rather
    than written so no dirty lines are written back during the timed call.
    block: the weights already on the device (the workload's x is drawn on
    its own seed). row_invariant: the call with that option (the block's
    own setting is restored afterwards). tiles: a new block of bf16 experts gets
    its tile-packed copy first. Algorithmic work: the MFMA flops of the routed and shared
    projections, and the bytes of the D distinct experts touched (as stored),
    the shared expert, the router weight, x and the bf16 output."""
    inp = W.generate(wl, experts=block is None)
    if block is None:
        block = lib.block_from_arrays(wl, inp)
        if tiles and wl.wfmt in ("bf16", "fp8"):
            block.pack_tiles()
    saved = block.row_invariant
    block.row_invariant = row_invariant
    x = lib.x_to_device(inp["x"])
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    buf = torch.ones(64 << 20, dtype=torch.int64, device="cuda") if flush else None
    warm(torch, lambda: block.forward(x, out=out, ids_out=ids))
    times = []
    for _ in range(steps):
        if buf is not None:
            buf.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        block.forward(x, out=out, ids_out=ids)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ups = []
    for _ in range(steps):
        if buf is not None:
            buf.sum()
        ev = lib.StageEvents()
        block.forward(x, out=out, ids_out=ids, events=ev)
        torch.cuda.synchronize()
        ups.append(ev.stage_ms())
    block.row_invariant = saved
    D = int(np.unique(ids.cpu().numpy()).size)
    eb_up, eb_down = expert_bytes(wl)
    algo = (D * (eb_up + eb_down) + shared_bytes(wl) + wl.E * wl.H * 4 +
            2 * wl.T * wl.H * 2)
    flops = sum(flops_of(wl))
    t = float(np.median(times)) * 1e-3
    gbs = algo / t / 1e9
    tfs = flops / t / 1e12
    return {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
            "act": wl.act, "weights": wl.wfmt, "I_shared": wl.I_shared,
            "distinct_experts": D, "us_per_step": 1e6 * t, "tokens_per_s": wl.T / t,
            "algorithmic_bytes": algo, "GBps": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
            "flops": flops, "tflops": tfs, "frac_bf16_peak": tfs / PEAK_BF16_TFLOPS,
            "cache_evicted": bool(flush), "row_invariant": bool(row_invariant),
            "tile_packed_weights": block.w_up_tiles is not None,
            "timing": "median of %d calls, one event pair each" % steps,
            "stages_us_with_events": {k: 1e3 * float(np.median([u[k] for u in ups]))
                                      for k in lib.STAGES}}


if __name__ == "__main__":
    main()
