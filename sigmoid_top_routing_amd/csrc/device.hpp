// device.hpp -- small device-side helpers shared by the library's kernels.
//
// Internal to libmoe; nothing outside sigmoid_top_routing_amd/csrc includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format;
// offsets are range checked against the record count, stride 0).
constexpr int kBufferWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from `base` + off into LDS at dst + 16 lane, through a
// raw buffer resource: offsets at or past 2^31 read zeros.
__device__ __forceinline__ void buffer_to_lds16(const void *base, uint4 *dst, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even, NaN stays NaN: gfx950's
// v_cvt_pk_bf16_f32 (one instruction for two values). Checked bit for bit
// against (u + 0x7fff + ((u >> 16) & 1)) >> 16 over all 2^32 fp32 inputs
// (NaN inputs give a NaN).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){lo, hi}, bf16x2_hw));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return pack_bf16x2(f, 0.0f) & 0xffffu;
}

// An OCP MX E8M0 scale byte as fp32: 2^(b - 127) (b = 0: 2^-127, a
// subnormal), 0xFF NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    const float v = b != 0 ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
    return b == 0xFFu ? __builtin_nanf("") : v;
}

// The four bytes of w, each two FP4 E2M1 codes (low nibble first), as four
// bf16 pairs: gfx950's v_cvt_scalef32_pk_bf16_fp4 with scale 1, which gives
// every E2M1 value exactly (checked on all 256 bytes in each byte position,
// -0 kept). The byte select is an immediate, hence the four spelled-out calls.
__device__ __forceinline__ void fp4_pairs(uint32_t w, uint32_t (&pr)[4]) {
    pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
}

// e^v in fp32 for v in [-17, 87]: v = n ln2 + r with n = rint(v log2 e)
// and a two-part ln2 (the high part has nine zero low bits), then the
// Taylor polynomial of e^r to degree 7 in Horner form and a scaling by 2^n.
// Used by the router's sigmoid, whose bits must not depend on a library.
__device__ __forceinline__ float exp_cw(float v) {
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    const float n = __builtin_rintf(v * log2e);
    float r = __builtin_fmaf(-n, ln2_hi, v);
    r = __builtin_fmaf(-n, ln2_lo, r);
    float p = 0x1.a01a02p-13f;                 // 1/5040
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f); // 1/720
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);  // 1/120
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);  // 1/24
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);  // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// Router score: 1 / (1 + e^-z), division correctly rounded (hipcc's default
// for fp32 '/'). NaN stays NaN; z > 17 gives 1 (the quotient rounds to 1
// there anyway); z < -87 gives 0, keeping every intermediate normal.
__device__ __forceinline__ float sigmoid_score(float z) {
    if (z != z)
        return z;
    if (z > 17.0f)
        return 1.0f;
    if (z < -87.0f)
        return 0.0f;
    return 1.0f / (1.0f + exp_cw(-z));
}

// Softmax router term e^d for d = z - (the row's largest logit) <= 0: 0
// below -87 (the sigmoid's tail rule), NaN stays NaN.
__device__ __forceinline__ float softmax_term(float d) {
    if (d != d)
        return d;
    if (d < -87.0f)
        return 0.0f;
    return exp_cw(d);
}

// SwiGLU epilogue: silu(g) * u with the hardware exp2 and reciprocal.
// Not bit-specified; held to the block's output tolerance.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 0x1.715476p+0f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// The same with GLM's swiglu_limit L when LIMIT (a separate instantiation,
// so the unlimited epilogue carries no extra instructions): g capped at L,
// u clamped to [-L, L], by comparisons, which keep a NaN.
template <bool LIMIT>
__device__ __forceinline__ float swiglu(float g, float u, float L) {
    if constexpr (LIMIT) {
        g = g > L ? L : g;
        u = u > L ? L : (u < -L ? -L : u);
    }
    return silu_mul(g, u);
}

// relu^2 epilogue: (u < 0 ? 0 : u)^2 in fp32; NaN and +inf pass through.
__device__ __forceinline__ float relu_sq(float u) {
    const float r = (u < 0.0f) ? 0.0f : u;
    return r * r;
}

// Top-k order key: larger key first, NaN below every number, +0 == -0.
__device__ __forceinline__ uint32_t order_key(float key) {
    if (key != key)
        return 0u;
    uint32_t u = __float_as_uint(key);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    const uint32_t lo = __shfl_xor((int)(uint32_t)v, mask, kWave);
    const uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), mask, kWave);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace moe
