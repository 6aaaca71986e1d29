"""CPU oracle of the sigmoid top-k routed MoE block (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this package. The product path (the HIP library and its binding) never
imports it, and it imports nothing from the product.
"""
from .oracle import (  # noqa: F401
    build, lib, activate, exp32, sigmoid32, softmax32, topk, route, plan, forward_tokens, affine4_decode,
    max_threads, add_rmsnorm, fp8_decode, fp4_decode, e8m0_decode, combine32, epilogue32, expert_rows32, SOURCE,
    LIBPATH,
)
