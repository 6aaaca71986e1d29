// route.hip -- router logits, sigmoid scores, bias-only top-k and weights.
//
// What is computed (TileGym PR #187, "Weight layout and routing"; TensorFold
// PR #1492, "What" and "Verification"):
//   z[t,e]   = sum_h x[t,h] * Wr[e,h], fp32, one fma per term, h ascending
//   s[t,e]   = 1 / (1 + e^-z)           (own exp, correctly rounded division)
//   key[t,e] = s[t,e] + bias[e]          (the bias only selects)
//   ids[t,:] = k experts by key, best first; ties to the lower index; NaN last
//   w[t,j]   = s[t,ids_j] / (sum_j s[t,ids_j] + eps)
//
// Layout on the device. A block has 4 waves. Each token's E experts are
// spread over LPT lanes (a power of two, at least 2), RE consecutive experts
// per lane,
// so one wave holds 64/LPT tokens. Per 32-wide slice of h the block stages
// x (as fp32, [h][token]) and Wr ([h][expert]) in LDS; a lane then runs RE
// independent fma chains, reading one broadcast x value and RE contiguous
// weights per h. Every chain keeps the sequential h order, so the logits are
// bit-identical to a plain loop. The top-k is k rounds of a 64-bit
// (order key, ~index) max over the token's LPT lanes with xor shuffles.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kHC = 32;      // h slice staged per step
constexpr int kThreads = 256;

template <int RE>
__global__ __launch_bounds__(kThreads) void k_route(const uint16_t *__restrict__ x,
                                                    const float *__restrict__ Wr,
                                                    const float *__restrict__ bias, int T, int H,
                                                    int E, int k, int LPT, int norm_topk,
                                                    float eps, int32_t *__restrict__ ids,
                                                    float *__restrict__ weights) {
    extern __shared__ float lds[];
    const int EP = LPT * RE;            // padded expert count
    const int TPW = kWave / LPT;        // tokens per wave
    const int TB = 4 * TPW;             // tokens per block
    float *ws = lds;                    // [kHC][EP]
    float *xs = lds + kHC * EP;         // [kHC][TB]

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int t0 = blockIdx.x * TB;
    const int tl = wave * TPW + lane / LPT;   // token within the block
    const int eg = lane % LPT;                // lane within the token's group
    const int e0 = eg * RE;

    float acc[RE];
#pragma unroll
    for (int r = 0; r < RE; ++r)
        acc[r] = 0.0f;

    for (int h0 = 0; h0 < H; h0 += kHC) {
        __syncthreads();
        for (int i = tid; i < EP * (kHC / 4); i += kThreads) {
            const int e = i % EP, q = i / EP;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E)
                v = *reinterpret_cast<const float4 *>(Wr + (size_t)e * H + h0 + 4 * q);
            ws[(4 * q + 0) * EP + e] = v.x;
            ws[(4 * q + 1) * EP + e] = v.y;
            ws[(4 * q + 2) * EP + e] = v.z;
            ws[(4 * q + 3) * EP + e] = v.w;
        }
        for (int i = tid; i < TB * (kHC / 8); i += kThreads) {
            const int j = i % TB, q = i / TB;
            const int t = t0 + j;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T)
                v = *reinterpret_cast<const uint4 *>(x + (size_t)t * H + h0 + 8 * q);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xs[(8 * q + 2 * c) * TB + j] = bf16_to_f32(w4[c] & 0xffffu);
                xs[(8 * q + 2 * c + 1) * TB + j] = bf16_to_f32(w4[c] >> 16);
            }
        }
        __syncthreads();
#pragma unroll 8
        for (int hh = 0; hh < kHC; ++hh) {
            const float xv = xs[hh * TB + tl];
            const float *wp = ws + hh * EP + e0;
#pragma unroll
            for (int r = 0; r < RE; ++r)
                acc[r] = __builtin_fmaf(xv, wp[r], acc[r]);
        }
    }

    // scores and keys; padded experts never win
    float s[RE];
    uint64_t cand[RE];
#pragma unroll
    for (int r = 0; r < RE; ++r) {
        const int e = e0 + r;
        s[r] = sigmoid_score(acc[r]);
        const float key = s[r] + (bias != nullptr && e < E ? bias[e] : 0.0f);
        cand[r] = (e < E) ? (((uint64_t)order_key(key) << 32) | (uint32_t)(0xffffu - e)) : 0ull;
    }

    int pick_e[8];
    float pick_s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pick_e[j] = 0;
        pick_s[j] = 0.0f;
        if (j < k) {
            uint64_t best = 0;
#pragma unroll
            for (int r = 0; r < RE; ++r)
                best = cand[r] > best ? cand[r] : best;
            for (int m = 1; m < LPT; m <<= 1) {
                const uint64_t o = shfl_xor_u64(best, m);
                best = o > best ? o : best;
            }
            const int e_win = 0xffff - (int)(best & 0xffffu);
            // the owning lane supplies the unbiased score and retires the pick
            float mine = 0.0f;
#pragma unroll
            for (int r = 0; r < RE; ++r) {
                if (e0 + r == e_win) {
                    mine = s[r];
                    cand[r] = 0ull;
                }
            }
            const int owner = (lane & ~(LPT - 1)) + e_win / RE;
            pick_e[j] = e_win;
            pick_s[j] = __shfl(mine, owner, kWave);
        }
    }

    const int t = t0 + tl;
    if (eg == 0 && t < T) {
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k)
                sum += pick_s[j];
        const float denom = sum + eps;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < k) {
                ids[(size_t)t * k + j] = pick_e[j];
                weights[(size_t)t * k + j] = norm_topk ? pick_s[j] / denom : pick_s[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const uint16_t *x, const float *Wr, const float *bias, int T, int H, int E,
                        int k, int norm_topk, float eps, int32_t *ids, float *weights,
                        hipStream_t stream) {
    if (T == 0)
        return hipSuccess;
    const int RE = E <= 16 ? 1 : E <= 64 ? 2 : E <= 128 ? 4 : 8;
    int LPT = 2;
    while (LPT * RE < E)
        LPT <<= 1;
    const int TB = 4 * (kWave / LPT);
    const int EP = LPT * RE;
    const size_t lds = sizeof(float) * kHC * (size_t)(EP + TB);
    const dim3 grid((T + TB - 1) / TB);
    switch (RE) {
    case 1:
        hipLaunchKernelGGL(k_route<1>, grid, dim3(kThreads), lds, stream, x, Wr, bias, T, H, E, k,
                           LPT, norm_topk, eps, ids, weights);
        break;
    case 2:
        hipLaunchKernelGGL(k_route<2>, grid, dim3(kThreads), lds, stream, x, Wr, bias, T, H, E, k,
                           LPT, norm_topk, eps, ids, weights);
        break;
    case 4:
        hipLaunchKernelGGL(k_route<4>, grid, dim3(kThreads), lds, stream, x, Wr, bias, T, H, E, k,
                           LPT, norm_topk, eps, ids, weights);
        break;
    default:
        hipLaunchKernelGGL(k_route<8>, grid, dim3(kThreads), lds, stream, x, Wr, bias, T, H, E, k,
                           LPT, norm_topk, eps, ids, weights);
        break;
    }
    return hipGetLastError();
}

}  // namespace moe
