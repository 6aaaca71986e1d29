"""Sigmoid top-k routed mixture-of-experts block for AMD Instinct MI355X (gfx950).

The block (router, expert plan, grouped expert GEMMs, weighted combine) runs
in hand-written HIP kernels behind a C ABI (include/moe.h); ``lib`` is the
Python binding and ``workloads`` the seeded synthetic inputs.
"""
