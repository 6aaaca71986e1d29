// norm.hip -- fused residual add + RMSNorm, the step that makes the block's
// input (TensorFold issue #548, the CUDA claim of the shared layer pieces:
// RMSNorm and the fused add + RMSNorm, a row's bits the same at every row
// count; TensorFold PR #1492, the reused addRmsTail norms).
//
//   r[c]            = h[t,c] + residual[t,c]     fp32 (r = residual without h)
//   residual_out[t] = bf16(r)                    round to nearest even
//   x[t,c]          = bf16(r[c] * inv * gamma[c]),  inv = 1 / sqrt(sum r^2 / H + eps)
//
// HBM-bound: per row it reads h and the residual and writes the residual and
// x, 8 H bytes (gamma stays in the caches). One wave per row, so a row's
// bits depend on nothing but the row: the wave holds the row in registers
// (8 columns per lane per pass of 512), adds its squares, reduces them by xor
// shuffles, and writes both outputs. Loads and stores go through a buffer
// resource spanning the row, so the columns past H of the last pass read
// zeros and their stores are dropped, with no branches between the loads.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kNormWaves = 4;   // rows per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(row), (short)0, bytes,
                                             kBufferWord3);
}

__device__ __forceinline__ void widen8(const uint4 &v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// NP passes of 512 columns (NP * 512 >= H).
template <int NP>
__global__ __launch_bounds__(kNormWaves * kWave) void k_add_rmsnorm(
    const uint16_t *__restrict__ h, const uint16_t *residual, const uint16_t *__restrict__ gamma,
    int T, int H, float eps, uint16_t *residual_out, uint16_t *__restrict__ x) {
    const int lane = threadIdx.x & (kWave - 1);
    // the row is the wave's: uniform, so the buffer resources stay scalar
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kNormWaves + threadIdx.x / kWave);
    if (t >= T)
        return;                                       // whole waves only
    const int row_bytes = H * 2;
    const size_t base = (size_t)t * H;
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(residual + base, row_bytes);
    const __amdgpu_buffer_rsrc_t rg = row_rsrc(gamma, row_bytes);
    float r[NP][8];
    uint4 hv[NP], rv[NP], gv[NP];
    const __amdgpu_buffer_rsrc_t rh = row_rsrc(h != nullptr ? h + base : residual + base,
                                              h != nullptr ? row_bytes : 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t off = (uint32_t)(p * 512 + lane * 8) * 2u;
        rv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
        hv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
        gv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
    }
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        float a[8], b[8];
        widen8(rv[p], a);
        widen8(hv[p], b);                             // zeros without h
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // without h, r is the residual itself (-0 + +0 would give +0)
            r[p][i] = h != nullptr ? a[i] + b[i] : a[i];
            ss = __builtin_fmaf(r[p][i], r[p][i], ss);
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        ss += __shfl_xor(ss, m, kWave);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)H + eps);
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + base, row_bytes);
    const __amdgpu_buffer_rsrc_t ro =
        row_rsrc(residual_out != nullptr ? residual_out + base : x + base,
                 residual_out != nullptr ? row_bytes : 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t off = (uint32_t)(p * 512 + lane * 8) * 2u;
        float g[8];
        widen8(gv[p], g);
        uint32_t xo[4], ro4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xo[i] = pack_bf16x2(r[p][2 * i] * inv * g[2 * i], r[p][2 * i + 1] * inv * g[2 * i + 1]);
            ro4[i] = pack_bf16x2(r[p][2 * i], r[p][2 * i + 1]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t,
                               make_uint4(xo[0], xo[1], xo[2], xo[3])), rx, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t,
                               make_uint4(ro4[0], ro4[1], ro4[2], ro4[3])), ro, off, 0, 0);
    }
}

template <int NP>
void launch_np(const uint16_t *h, const uint16_t *residual, const uint16_t *gamma, int T, int H,
               float eps, uint16_t *residual_out, uint16_t *x, hipStream_t stream) {
    const dim3 grid((T + kNormWaves - 1) / kNormWaves);
    hipLaunchKernelGGL(k_add_rmsnorm<NP>, grid, dim3(kNormWaves * kWave), 0, stream, h, residual,
                       gamma, T, H, eps, residual_out, x);
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t *h, const uint16_t *residual, const uint16_t *gamma,
                              int T, int H, float eps, uint16_t *residual_out, uint16_t *x,
                              hipStream_t stream) {
    if (T == 0)
        return hipSuccess;
    if (H % 64 != 0 || H > kNormMaxH)
        return hipErrorInvalidValue;
    const int passes = (H + 511) / 512;
    if (passes <= 1)
        launch_np<1>(h, residual, gamma, T, H, eps, residual_out, x, stream);
    else if (passes <= 2)
        launch_np<2>(h, residual, gamma, T, H, eps, residual_out, x, stream);
    else if (passes <= 4)
        launch_np<4>(h, residual, gamma, T, H, eps, residual_out, x, stream);
    else if (passes <= 8)
        launch_np<8>(h, residual, gamma, T, H, eps, residual_out, x, stream);
    else
        launch_np<16>(h, residual, gamma, T, H, eps, residual_out, x, stream);
    return hipGetLastError();
}

}  // namespace moe
