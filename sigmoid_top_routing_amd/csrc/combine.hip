// combine.hip -- weighted combine back to token order plus the shared expert.
//
//   acc = 0; acc = fma(w[t,j], y[slot_of[t*k+j], h], acc) for j = 0..k-1 (ascending)
//   acc = acc * routed_scale          (the routed sum is scaled once, here)
//   acc = acc + shared[t, h]          (the shared expert is added unscaled)
// When the shared expert ran as m plan segments of the routed experts' width
// (I_shared = m I), its output is the sum of m partial rows, added first in
// ascending order: s = shared_0[t, h] + ... + shared_{m-1}[t, h], acc + s.
//   out[t, h] = round(acc)            (bf16 nearest-even, or fp32 as is)
// vllm.cpp PR #684 (W2 commit): the routed scale multiplies the finished
// routed sum before the shared output is added; folding it into each weight
// rounds k times instead of once and gives different bits. TileGym PR #187
// ("Weight layout and routing"): the routed scaling factor comes after the
// normalised weights.
//
// With fold (Laguna's order, only without a shared expert) the scale goes
// into each weight instead: acc = fma(routed_scale * w[t,j], y, acc), j
// ascending, and nothing after; the product is rounded once per term, so the
// bits differ from the order above (vllm.cpp PR #684, the review-repairs
// commit). A separate instantiation, so the default order's code is unchanged.
//
// y holds the down projection's rows in segment order (assignment a at row
// slot_of[a], the plan's position), so the expert kernels write whole rows
// where their tiles are and the combine gathers a token's k rows. Each
// thread produces 8 consecutive outputs of one token: k 32-byte reads of y
// and one 16-byte (bf16) or 32-byte (fp32) store, all coalesced.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

template <bool FOLD>
__global__ __launch_bounds__(kThreads) void k_combine(const float *__restrict__ y,
                                                      const int32_t *__restrict__ slot,
                                                      const float *__restrict__ w,
                                                      const float *__restrict__ shared,
                                                      int shared_terms, int T, int H, int k,
                                                      float rsf, void *out, int out_f32) {
    const int per_tok = H / 8;
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (size_t)T * per_tok)
        return;
    const int t = (int)(idx / per_tok);
    const int h0 = (int)(idx % per_tok) * 8;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
        acc[c] = 0.0f;
    for (int j = 0; j < k; ++j) {
        const float wj = FOLD ? rsf * w[(size_t)t * k + j] : w[(size_t)t * k + j];
        const int row = slot[(size_t)t * k + j];
        const float4 *yp = reinterpret_cast<const float4 *>(y + (size_t)row * H + h0);
        const float4 a = yp[0], b = yp[1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_fmaf(wj, v[c], acc[c]);
    }
    if (!FOLD) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = acc[c] * rsf;
    }
    if (shared != nullptr) {
        float s[8];
        for (int v = 0; v < shared_terms; ++v) {
            const float4 *sp =
                reinterpret_cast<const float4 *>(shared + ((size_t)v * T + t) * H + h0);
            const float4 a = sp[0], b = sp[1];
            const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int c = 0; c < 8; ++c)
                s[c] = v == 0 ? e[c] : s[c] + e[c];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = acc[c] + s[c];
    }
    if (out_f32) {
        float4 *op = reinterpret_cast<float4 *>((float *)out + (size_t)t * H + h0);
        op[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        op[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        uint4 v = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        *reinterpret_cast<uint4 *>((uint16_t *)out + (size_t)t * H + h0) = v;
    }
}

}  // namespace

hipError_t launch_combine(const float *y_seg, const int32_t *slot_of, const float *weights,
                          const float *shared, int shared_terms, int T, int H, int k,
                          float routed_scale, bool fold, void *out, int out_f32,
                          hipStream_t stream) {
    const size_t n = (size_t)T * (H / 8);
    if (n == 0)
        return hipSuccess;
    if (shared != nullptr && shared_terms < 1)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (fold)
        hipLaunchKernelGGL(k_combine<true>, grid, dim3(kThreads), 0, stream, y_seg, slot_of,
                           weights, shared, shared_terms, T, H, k, routed_scale, out, out_f32);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, dim3(kThreads), 0, stream, y_seg, slot_of,
                           weights, shared, shared_terms, T, H, k, routed_scale, out, out_f32);
    return hipGetLastError();
}

}  // namespace moe
