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
// Two launches.
//
// k_logits is a small fp32 GEMM, z = x Wr^T, over (token tile x expert
// tile) workgroups spread across the chip: one CU streams only a few tens of
// GB/s, so no workgroup may reload the whole router weight for a handful of
// tokens. A thread owns RT tokens x RE experts (independent fma chains that
// hide the fma latency); its experts are e0 + et + r*ET so that neighbouring
// lanes read neighbouring LDS rows. H is walked in chunks: Wr ([expert][h])
// and x (fp32, [token][h]) for a chunk are staged in LDS with 16-byte row
// padding, double buffered, and the next chunk's coalesced global loads are
// issued before the current chunk's fmas. Per four h a thread reads one
// float4 per token and per expert and issues 4*RT*RE fmas; every chain runs
// in sequential h order, so z is bit-identical to a plain loop.
//
// k_topk reads z, applies the sigmoid and the bias, and picks the top k of
// each token with k rounds of a 64-bit (order key, ~index) max over the
// token's lanes (xor shuffles); then the weights. When one workgroup holds
// every token (decode-sized batches) it also builds the plan.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kMaxThreads = 256;
constexpr int kMaxW = 12;      // float4 router-weight prefetch slots per thread
constexpr int kMaxX = 8;       // uint4 (8 x bf16) x prefetch slots per thread
constexpr int kLdsBudget = 100 * 1024;
constexpr int kRing = 8;       // groups of four h read from LDS ahead of their fmas

template <int RT, int RE>
__global__ __launch_bounds__(kMaxThreads) void k_logits(const uint16_t *__restrict__ x,
                                                        const float *__restrict__ Wr, int T,
                                                        int H, int E, int TT, int ET, int HC,
                                                        float *__restrict__ z) {
    extern __shared__ float lds[];
    const int nthr = kMaxThreads;            // every thread stages, TT * ET compute
    const int TB = TT * RT;                  // tokens per tile
    const int EB = ET * RE;                  // experts per tile
    const int HP = HC + 4;                   // padded LDS row
    float *const wbuf = lds;                 // [2][EB][HP]
    float *const xbuf = lds + 2 * EB * HP;   // [2][TB][HP]

    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * TB;
    const int e0 = blockIdx.y * EB;
    const int tt = tid / ET;
    const int et = tid % ET;

    float4 wreg[kMaxW];
    uint4 xreg[kMaxX];
    auto load = [&](int h0, int hc) {
        const int qw = hc / 4, qx = hc / 8;
        const int nw = EB * qw, nx = TB * qx;
#pragma unroll
        for (int i = 0; i < kMaxW; ++i) {
            const int idx = tid + i * nthr;
            if (idx < nw) {
                const int e = e0 + idx / qw, q = idx % qw;
                wreg[i] = e < E ? *reinterpret_cast<const float4 *>(Wr + (size_t)e * H + h0 + 4 * q)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxX; ++i) {
            const int idx = tid + i * nthr;
            if (idx < nx) {
                const int t = t0 + idx / qx, q = idx % qx;
                xreg[i] = t < T ? *reinterpret_cast<const uint4 *>(x + (size_t)t * H + h0 + 8 * q)
                                : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store = [&](int buf, int hc) {
        float *ws = wbuf + buf * EB * HP;
        float *xs = xbuf + buf * TB * HP;
        const int qw = hc / 4, qx = hc / 8;
        const int nw = EB * qw, nx = TB * qx;
#pragma unroll
        for (int i = 0; i < kMaxW; ++i) {
            const int idx = tid + i * nthr;
            if (idx < nw)
                *reinterpret_cast<float4 *>(ws + (idx / qw) * HP + 4 * (idx % qw)) = wreg[i];
        }
#pragma unroll
        for (int i = 0; i < kMaxX; ++i) {
            const int idx = tid + i * nthr;
            if (idx < nx) {
                float *row = xs + (idx / qx) * HP + 8 * (idx % qx);
                const uint4 v = xreg[i];
                *reinterpret_cast<float4 *>(row) =
                    make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                                bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16));
                *reinterpret_cast<float4 *>(row + 4) =
                    make_float4(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16),
                                bf16_to_f32(v.w & 0xffffu), bf16_to_f32(v.w >> 16));
            }
        }
    };

    float acc[RT][RE];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int r = 0; r < RE; ++r)
            acc[i][r] = 0.0f;
    const bool computes = tid < TT * ET;

    int hc = H < HC ? H : HC;
    load(0, hc);
    int buf = 0;
    for (int h0 = 0; h0 < H; h0 += HC) {
        store(buf, hc);
        __syncthreads();
        const int hn = h0 + HC;
        const int hc_next = H - hn < HC ? H - hn : HC;
        if (hn < H)
            load(hn, hc_next);
        if (computes) {
            const float *xs = xbuf + buf * TB * HP + (tt * RT) * HP;
            const float *ws = wbuf + buf * EB * HP + et * HP;
            // blocks of 4 * kRing h: every LDS read of a block is issued
            // first, then its fmas (chains in h order), so the read latency
            // is paid once per block and overlaps the first fmas
            for (int hh0 = 0; hh0 < hc; hh0 += 4 * kRing) {
                float4 xv[kRing][RT], wv[kRing][RE];
#pragma unroll
                for (int d = 0; d < kRing; ++d) {
#pragma unroll
                    for (int i = 0; i < RT; ++i)
                        xv[d][i] = *reinterpret_cast<const float4 *>(xs + i * HP + hh0 + 4 * d);
#pragma unroll
                    for (int r = 0; r < RE; ++r)
                        wv[d][r] = *reinterpret_cast<const float4 *>(ws + r * ET * HP + hh0 + 4 * d);
                }
#pragma unroll
                for (int d = 0; d < kRing; ++d)
#pragma unroll
                    for (int i = 0; i < RT; ++i)
#pragma unroll
                        for (int r = 0; r < RE; ++r) {
                            float a = acc[i][r];
                            a = __builtin_fmaf(xv[d][i].x, wv[d][r].x, a);
                            a = __builtin_fmaf(xv[d][i].y, wv[d][r].y, a);
                            a = __builtin_fmaf(xv[d][i].z, wv[d][r].z, a);
                            a = __builtin_fmaf(xv[d][i].w, wv[d][r].w, a);
                            acc[i][r] = a;
                        }
            }
        }
        hc = hc_next;
        buf ^= 1;
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = t0 + tt * RT + i;
#pragma unroll
        for (int r = 0; r < RE; ++r) {
            const int e = e0 + et + r * ET;
            if (computes && t < T && e < E)
                z[(size_t)t * E + e] = acc[i][r];
        }
    }
}

template <int RE>
__global__ __launch_bounds__(kMaxThreads) void k_topk(const float *__restrict__ z,
                                                      const float *__restrict__ bias, int T,
                                                      int E, int k, int LPT, int norm_topk,
                                                      float eps, int32_t *__restrict__ ids,
                                                      float *__restrict__ weights, PlanOut plan) {
    __shared__ int s_ids[kFusedPlanMaxA];
    __shared__ int s_cnt[256];
    __shared__ int s_off[256];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int per_block = kMaxThreads / LPT;
    const int tb = tid / LPT;                   // token within the block
    const int t = blockIdx.x * per_block + tb;
    const int eg = tid % LPT;                   // experts eg + r * LPT

    float s[RE];
    uint64_t cand[RE];
#pragma unroll
    for (int r = 0; r < RE; ++r) {
        const int e = eg + r * LPT;
        const bool real = t < T && e < E;
        s[r] = real ? sigmoid_score(z[(size_t)t * E + e]) : 0.0f;
        const float key = s[r] + (bias != nullptr && real ? bias[e] : 0.0f);
        cand[r] = real ? (((uint64_t)order_key(key) << 32) | (uint32_t)(0xffffu - e)) : 0ull;
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
                if (eg + r * LPT == e_win) {
                    mine = s[r];
                    cand[r] = 0ull;
                }
            }
            pick_e[j] = e_win;
            pick_s[j] = __shfl(mine, (lane & ~(LPT - 1)) + e_win % LPT, kWave);
        }
    }
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
                if (plan.counts != nullptr)
                    s_ids[tb * k + j] = pick_e[j];
            }
        }
    }
    if (plan.counts == nullptr)
        return;

    // One block holds every token: it also builds the plan (histogram,
    // exclusive scan, stable scatter), saving two launches on decode steps.
    __syncthreads();
    const int A = T * k;
    if (tid < E) {
        int c = 0;
        for (int a = 0; a < A; ++a)
            c += s_ids[a] == tid;
        s_cnt[tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            s_off[e] = run;
            plan.counts[e] = s_cnt[e];
            plan.offsets[e] = run;
            run += s_cnt[e];
        }
        plan.offsets[E] = run;
    }
    __syncthreads();
    if (tid < E) {
        int pos = s_off[tid];
        for (int a = 0; a < A; ++a) {
            if (s_ids[a] == tid) {
                plan.sorted[pos] = a;
                plan.slot_of[a] = pos;
                ++pos;
            }
        }
    }
}

template <int RT, int RE>
void launch_logits(dim3 grid, size_t lds, hipStream_t stream, const uint16_t *x,
                   const float *Wr, int T, int H, int E, int TT, int ET, int HC, float *z) {
    static const bool opt_in = [] {
        (void)hipFuncSetAttribute((const void *)k_logits<RT, RE>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
        return true;
    }();
    (void)opt_in;
    hipLaunchKernelGGL((k_logits<RT, RE>), grid, dim3(kMaxThreads), lds, stream, x, Wr, T, H, E,
                       TT, ET, HC, z);
}

struct LogitsTiling {
    int RT, RE, TT, ET, HC;
    size_t lds;
    dim3 grid;
};

// Tile choice. Few tokens: four experts per workgroup and one chain per
// lane, so the (sequential) chains run side by side on E/4 CUs, each of
// which stages a whole row range at once. Many tokens: 32 experts per tile
// and as many tokens as keep about one workgroup per CU, with 2 to 4 chains
// per lane.
LogitsTiling choose_tiling(int T, int H, int E) {
    LogitsTiling c{};
    const int cus = 256;
    if (T <= 64) {
        c.RT = 1;
        c.RE = 1;
        c.ET = 4;
        c.TT = 64;
        while (c.TT / 2 >= T && c.TT > 1)
            c.TT /= 2;
    } else {
        c.ET = E >= 32 ? 32 : (E >= 16 ? 16 : 8);
        c.RE = 1;
        const int etiles = (E + c.ET - 1) / c.ET;
        const int TT = 256 / c.ET;
        // tokens per tile so that tiles ~ CUs, 1..4 per thread
        const int want_tb = (int)(((int64_t)T * etiles + cus - 1) / cus);
        c.RT = want_tb >= 4 * TT ? 4 : want_tb >= 2 * TT ? 2 : 1;
        c.TT = TT;
    }
    const int TB = c.TT * c.RT, EB = c.ET * c.RE;
    auto fits = [&](int hc) {
        return (size_t)2 * sizeof(float) * (EB + TB) * (hc + 4) <= (size_t)kLdsBudget &&
               EB * hc <= kMaxW * 4 * kMaxThreads && TB * hc <= kMaxX * 8 * kMaxThreads;
    };
    // the whole of H in one chunk when it fits (one load round trip)
    c.HC = 4096;
    while (c.HC > 8 && !fits(c.HC))
        c.HC >>= 1;
    c.lds = (size_t)2 * sizeof(float) * (EB + TB) * (c.HC + 4);
    c.grid = dim3((T + TB - 1) / TB, (E + EB - 1) / EB);
    return c;
}

}  // namespace

size_t route_scratch_bytes(int T, int E) { return (size_t)T * E * sizeof(float); }

hipError_t launch_route(const uint16_t *x, const float *Wr, const float *bias, int T, int H, int E,
                        int k, int norm_topk, float eps, int32_t *ids, float *weights,
                        float *z_scratch, PlanOut plan, bool *plan_done, hipStream_t stream) {
    if (plan_done != nullptr)
        *plan_done = false;
    if (T == 0)
        return hipSuccess;
    const LogitsTiling c = choose_tiling(T, H, E);
    // H is a multiple of 64 and a chunk is a power of two >= 64 (or all of
    // H), so every chunk is a whole number of ring turns (4 * kRing wide)
    if (c.HC < 4 * kRing || H % 64 != 0 || c.TT * c.ET > kMaxThreads)
        return hipErrorInvalidValue;
    const int key = c.RT * 10 + c.RE;
    switch (key) {
    case 11:
        launch_logits<1, 1>(c.grid, c.lds, stream, x, Wr, T, H, E, c.TT, c.ET, c.HC, z_scratch);
        break;
    case 21:
        launch_logits<2, 1>(c.grid, c.lds, stream, x, Wr, T, H, E, c.TT, c.ET, c.HC, z_scratch);
        break;
    case 41:
        launch_logits<4, 1>(c.grid, c.lds, stream, x, Wr, T, H, E, c.TT, c.ET, c.HC, z_scratch);
        break;
    default:
        return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;

    // top-k: a token's experts are spread over LPT lanes, RE per lane
    const int RE = E > 128 ? 4 : E > 64 ? 2 : 1;
    int LPT = 2;
    while (LPT * RE < E)
        LPT <<= 1;
    const int per_block = kMaxThreads / LPT;
    const dim3 grid((T + per_block - 1) / per_block);
    const bool fuse = plan.counts != nullptr && grid.x == 1 && T * k <= kFusedPlanMaxA;
    if (!fuse)
        plan = PlanOut{};
    switch (RE) {
    case 1:
        hipLaunchKernelGGL(k_topk<1>, grid, dim3(kMaxThreads), 0, stream, z_scratch, bias, T, E,
                           k, LPT, norm_topk, eps, ids, weights, plan);
        break;
    case 2:
        hipLaunchKernelGGL(k_topk<2>, grid, dim3(kMaxThreads), 0, stream, z_scratch, bias, T, E,
                           k, LPT, norm_topk, eps, ids, weights, plan);
        break;
    default:
        hipLaunchKernelGGL(k_topk<4>, grid, dim3(kMaxThreads), 0, stream, z_scratch, bias, T, E,
                           k, LPT, norm_topk, eps, ids, weights, plan);
        break;
    }
    err = hipGetLastError();
    if (err == hipSuccess && plan_done != nullptr)
        *plan_done = fuse;
    return err;
}

}  // namespace moe
