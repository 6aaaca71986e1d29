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
// Two launches, or one for decode-sized batches (k_route_decode).
//
// k_logits computes z = x Wr^T as T*E independent fma chains of length H,
// each in h order (see the kernel for the layout). The chains are what
// bound it: at the prefill shapes they fill the chip's fp32 lanes, at a
// decode step they are latency-bound, and k_logits_few takes that case.
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

// k_logits: one lane per token, C experts per wave (C chains per lane).
// A workgroup of 4 waves owns 64 tokens and 4*C experts and walks H in
// chunks of kHC. Per chunk it stages the 64 token rows, converted once to
// fp32 for the four waves that share them (a lane reads 4 of its own h per
// 16-byte LDS read; rows are padded by 16 bytes so the 16 lanes of a pass
// hit distinct banks), and the experts' router rows (every lane of a wave
// reads the same address: one broadcast per 4 h and expert). The next
// chunk's global loads are issued before the current chunk's fmas and
// written to the other LDS buffer after them; within a chunk the LDS reads
// of the next 16 h are issued before the fmas of the current 16. Every
// chain runs in h order, so z is bit-identical to a plain loop over h.
constexpr int kTok = 64;                 // tokens per workgroup (one per lane)
constexpr int kHC = 256;                 // h per LDS chunk
constexpr int kXRow = kHC / 4 + 1;       // float4 per staged token row (+ pad)
constexpr int kWRow = kHC / 4 + 1;       // float4 per staged router row (+ pad)
constexpr int kXLoads = kTok * (kHC / 8) / kMaxThreads;   // uint4 x loads per thread

template <int C>
__global__ __launch_bounds__(kMaxThreads) void k_logits(const uint16_t *__restrict__ x,
                                                        const float *__restrict__ Wr, int T,
                                                        int H, int E, float *__restrict__ z) {
    constexpr int EB = 4 * C;                                  // experts per workgroup
    constexpr int WLOADS = (EB * (kHC / 4) + kMaxThreads - 1) / kMaxThreads;
    __shared__ float4 xs[2][kTok * kXRow];
    __shared__ float4 ws[2][EB * kWRow];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int t0 = blockIdx.x * kTok;
    const int e0 = blockIdx.y * EB;

    uint4 xreg[kXLoads];
    float4 wreg[WLOADS];
    // chunk h0 .. h0 + hc - 1 (hc a multiple of 64) into registers
    auto load = [&](int h0, int hc) {
        const int q = hc / 8;                                  // uint4 per token row
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int idx = tid + i * kMaxThreads;
            const int r = idx / (kHC / 8), c = idx % (kHC / 8);
            const int t = t0 + r;
            xreg[i] = (t < T && c < q) ? *reinterpret_cast<const uint4 *>(x + (size_t)t * H + h0 + 8 * c)
                                       : make_uint4(0, 0, 0, 0);
        }
        const int qw = hc / 4;
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const int idx = tid + i * kMaxThreads;
            const int r = idx / (kHC / 4), c = idx % (kHC / 4);
            const int e = e0 + r;
            wreg[i] = (r < EB && e < E && c < qw)
                          ? *reinterpret_cast<const float4 *>(Wr + (size_t)e * H + h0 + 4 * c)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int idx = tid + i * kMaxThreads;
            float4 *row = xs[buf] + (idx / (kHC / 8)) * kXRow + 2 * (idx % (kHC / 8));
            const uint4 v = xreg[i];
            row[0] = make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                                 bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16));
            row[1] = make_float4(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16),
                                 bf16_to_f32(v.w & 0xffffu), bf16_to_f32(v.w >> 16));
        }
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const int idx = tid + i * kMaxThreads;
            if (idx / (kHC / 4) < EB)
                ws[buf][(idx / (kHC / 4)) * kWRow + idx % (kHC / 4)] = wreg[i];
        }
    };

    float acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
        acc[c] = 0.0f;
    // 16 h: x[i] holds h 4i..4i+3 of this lane's token, w[c][i] the same h
    // of expert c
    // (the chains alternate instruction by instruction: in-order issue then
    // never waits on the previous fma of the same chain)
    auto fma16 = [&](const float4 (&xv)[4], const float4 (&wv)[C][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int c = 0; c < C; ++c)
                acc[c] = __builtin_fmaf(xv[i].x, wv[c][i].x, acc[c]);
#pragma unroll
            for (int c = 0; c < C; ++c)
                acc[c] = __builtin_fmaf(xv[i].y, wv[c][i].y, acc[c]);
#pragma unroll
            for (int c = 0; c < C; ++c)
                acc[c] = __builtin_fmaf(xv[i].z, wv[c][i].z, acc[c]);
#pragma unroll
            for (int c = 0; c < C; ++c)
                acc[c] = __builtin_fmaf(xv[i].w, wv[c][i].w, acc[c]);
        }
    };

    int hc = H < kHC ? H : kHC;
    load(0, hc);
    int buf = 0;
    for (int h0 = 0; h0 < H; h0 += kHC) {
        store(buf);
        __syncthreads();
        const int hn = h0 + kHC;
        const int hc_next = H - hn < kHC ? H - hn : kHC;
        if (hn < H)
            load(hn, hc_next);
        const float4 *xr = xs[buf] + lane * kXRow;
        const float4 *wr = ws[buf] + (wave * C) * kWRow;
        float4 xa[4], xb[4];
        float4 wa[C][4], wb[C][4];
        auto read16 = [&](int g, float4 (&xv)[4], float4 (&wv)[C][4]) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xv[i] = xr[4 * g + i];
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wv[c][i] = wr[c * kWRow + 4 * g + i];
        };
        const int groups = hc / 16;          // hc is a multiple of 64: even
        read16(0, xa, wa);
        for (int g = 0; g < groups; g += 2) {
            read16(g + 1, xb, wb);
            __builtin_amdgcn_sched_barrier(0);
            fma16(xa, wa);
            __builtin_amdgcn_sched_barrier(0);
            read16(g + 2 < groups ? g + 2 : g + 1, xa, wa);   // no branch: no copies
            __builtin_amdgcn_sched_barrier(0);
            fma16(xb, wb);
            __builtin_amdgcn_sched_barrier(0);
        }
        hc = hc_next;
        buf ^= 1;
        __syncthreads();                    // the buffer refilled next is no longer read
    }
    const int t = t0 + lane;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = e0 + wave * C + c;
        if (t < T && e < E)
            z[(size_t)t * E + e] = acc[c];
    }
}

// k_logits_ring: the same lanes and chains as k_logits<2> (a lane per token,
// two experts per wave: 64 tokens and 8 experts per workgroup), for H a
// multiple of 128. The operands come in by range-checked buffer loads
// straight into a ring of 4 LDS stages of 128 h (x as bf16, the router rows
// as fp32), requested three stages ahead, so the chains do not wait on
// memory once the ring is full; no registers hold staged data. A token row's
// 16-byte pieces (8 h) sit at piece c ^ (t % 16) of its LDS row, so the 16
// lanes of a 16-byte read hit distinct banks; the router rows are read by
// every lane at once (broadcast). Every chain still runs in h order.
constexpr int kRingH = 128;
constexpr int kRingStages = 4;
constexpr int kRingX = kTok * (kRingH / 8);             // 16-byte x pieces per stage
constexpr int kRingW = 8 * (kRingH / 4);                // 16-byte router pieces per stage
constexpr int kRingStage = kRingX + kRingW;             // 20 KB
constexpr int kRingPer = kRingStage / kMaxThreads;      // requests per thread per stage
constexpr uint32_t kRingPast = 0x80000000u;             // an offset that reads zeros

// One stage: the chains over stage S (128 h); the refill of stage F with h
// block sf (none when sf < 0). One call site, so the LDS reads of S and the
// loads into F share one alias scope and the compiler does not order the
// reads behind loads still in flight; the caller's waits do that.
__device__ __forceinline__ void ring_stage(const uint4 *__restrict__ S, uint4 *__restrict__ F,
                                           const uint16_t *x, const float *Wr,
                                           const uint32_t (&xoff)[kRingPer - 1], uint32_t woff,
                                           int sf, float &acc0, float &acc1) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (sf >= 0) {
#pragma unroll
        for (int q = 0; q < kRingPer - 1; ++q)
            buffer_to_lds16(x, F + (q * 4 + wave) * kWave, xoff[q] + sf * (kRingH * 2));
        buffer_to_lds16(Wr, F + kRingX + wave * kWave, woff + sf * (kRingH * 4));
    }
    const int t = lane;
    const uint4 *xrow = S + t * (kRingH / 8);
    const float4 *wa = reinterpret_cast<const float4 *>(S + kRingX) + (2 * wave) * (kRingH / 4);
    const float4 *wb = wa + kRingH / 4;
    // 8 h per group: one 16-byte x piece, two float4 of each router row
    auto read = [&](int g, uint4 &xv, float4 (&av)[2], float4 (&bv)[2]) {
        xv = xrow[g ^ (t & 15)];
        av[0] = wa[2 * g];
        av[1] = wa[2 * g + 1];
        bv[0] = wb[2 * g];
        bv[1] = wb[2 * g + 1];
    };
    auto fma8 = [&](const uint4 &xv, const float4 (&av)[2], const float4 (&bv)[2]) {
        const float xs[8] = {bf16_to_f32(xv.x & 0xffffu), bf16_to_f32(xv.x >> 16),
                             bf16_to_f32(xv.y & 0xffffu), bf16_to_f32(xv.y >> 16),
                             bf16_to_f32(xv.z & 0xffffu), bf16_to_f32(xv.z >> 16),
                             bf16_to_f32(xv.w & 0xffffu), bf16_to_f32(xv.w >> 16)};
        const float as[8] = {av[0].x, av[0].y, av[0].z, av[0].w, av[1].x, av[1].y, av[1].z, av[1].w};
        const float bs[8] = {bv[0].x, bv[0].y, bv[0].z, bv[0].w, bv[1].x, bv[1].y, bv[1].z, bv[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc0 = __builtin_fmaf(xs[i], as[i], acc0);
            acc1 = __builtin_fmaf(xs[i], bs[i], acc1);
        }
    };
    uint4 xa, xb;
    float4 aa[2], ba[2], ab[2], bb[2];
    constexpr int G = kRingH / 8;                           // 16 groups, even
    read(0, xa, aa, ba);
#pragma unroll
    for (int g = 0; g < G; g += 2) {
        read(g + 1, xb, ab, bb);
        __builtin_amdgcn_sched_barrier(0);
        fma8(xa, aa, ba);
        __builtin_amdgcn_sched_barrier(0);
        if (g + 2 < G)
            read(g + 2, xa, aa, ba);
        __builtin_amdgcn_sched_barrier(0);
        fma8(xb, ab, bb);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(kMaxThreads) void k_logits_ring(const uint16_t *__restrict__ x,
                                                             const float *__restrict__ Wr, int T,
                                                             int H, int E, float *__restrict__ z) {
    __shared__ uint4 ring[kRingStages * kRingStage];    // 80 KB
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int t0 = blockIdx.x * kTok;
    const int e0 = blockIdx.y * 8;
    const int S = H / kRingH;
    // byte offsets of this thread's pieces in h block 0; rows past T or E
    // read zeros
    uint32_t xoff[kRingPer - 1];
#pragma unroll
    for (int q = 0; q < kRingPer - 1; ++q) {
        const int pos = (q * 4 + wave) * kWave + lane;     // LDS piece
        const int r = pos / (kRingH / 8), c = (pos % (kRingH / 8)) ^ (r & 15);
        xoff[q] = t0 + r < T ? ((uint32_t)(t0 + r) * (uint32_t)H + 8u * c) * 2u : kRingPast;
    }
    uint32_t woff;
    {
        const int pos = wave * kWave + lane;
        const int j = pos / (kRingH / 4), c = pos % (kRingH / 4);
        woff = e0 + j < E ? ((uint32_t)(e0 + j) * (uint32_t)H + 4u * c) * 4u : kRingPast;
    }
    // the first three stages
#pragma unroll
    for (int s = 0; s < kRingStages - 1; ++s) {
        if (s < S) {
            uint4 *F = ring + s * kRingStage;
#pragma unroll
            for (int q = 0; q < kRingPer - 1; ++q)
                buffer_to_lds16(x, F + (q * 4 + wave) * kWave, xoff[q] + s * (kRingH * 2));
            buffer_to_lds16(Wr, F + kRingX + wave * kWave, woff + s * (kRingH * 4));
        }
    }
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int s = 0; s < S; ++s) {
        // stage s is in once at most the requests of the two stages after
        // it are still in flight (fewer near the end)
        if (s + 2 < S)
            wait_vmcnt<2 * kRingPer>();
        else if (s + 1 < S)
            wait_vmcnt<kRingPer>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();       // every wave's pieces are in; stage s - 1 is read
        ring_stage(ring + (s & 3) * kRingStage, ring + ((s + 3) & 3) * kRingStage, x, Wr, xoff,
                   woff, s + 3 < S ? s + 3 : -1, acc0, acc1);
    }
    const int t = t0 + lane;
    const int e = e0 + 2 * wave;
    if (t < T) {
        if (e < E)
            z[(size_t)t * E + e] = acc0;
        if (e + 1 < E)
            z[(size_t)t * E + e + 1] = acc1;
    }
}

// k_logits_few: decode-sized batches (T <= 8, H <= 2048). The chains are
// the whole cost there (H dependent fmas each), so the point is to start
// them early and never stall them: a workgroup owns 8 experts and every
// token, requests all of its rows at once (four h-quarters, in order), and
// moves quarter q to LDS (x converted to fp32) as soon as it has landed;
// lanes 0..15 of each wave then run the chains of 2 experts x 8 tokens over
// that quarter, reading 16 h ahead. Rows are padded by 16 bytes, so the 8
// token rows read together sit in distinct banks.
constexpr int kFewT = 8;
constexpr int kFewE = 8;
constexpr int kFewMaxH = 2048;
constexpr int kFewRow = kFewMaxH / 4 + 1;          // float4 per staged row (+ pad)

__global__ __launch_bounds__(kMaxThreads) void k_logits_few(const uint16_t *__restrict__ x,
                                                            const float *__restrict__ Wr, int T,
                                                            int H, int E, float *__restrict__ z) {
    __shared__ float4 xs[kFewT * kFewRow];
    __shared__ float4 ws[kFewE * kFewRow];
    __shared__ float4 junk[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int e0 = blockIdx.x * kFewE;
    const int hq = H / 4;                           // h per quarter, a multiple of 16
    const int rs = hq + 1;                          // float4 per staged row
    // loader: 32 threads per row; row r = tid / 32. Buffer loads return
    // zeros past the end of x or Wr (and for the offset pushed there when a
    // piece lies outside the quarter), so every load is issued
    // unconditionally and the quarters can be waited for one at a time.
    const int lr = tid / 32, lc = tid % 32;
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, T * H * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)Wr, (short)0, E * H * 4, kBufferWord3);
    const uint32_t kPast = 0x80000000u;
    uint4 xr[4][2];
    float4 wr[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = lc + 32 * i;              // uint4 of the quarter's row
            const uint32_t off = q < hq / 8 ? (uint32_t)(lr * H + c * hq + 8 * q) * 2u : kPast;
            xr[c][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lc + 32 * i;              // float4 of the quarter's row
            const uint32_t off =
                q < hq / 4 ? (uint32_t)((e0 + lr) * H + c * hq + 4 * q) * 4u : kPast;
            wr[c][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0));
        }
    }
    const int t = lane & 7;
    const int j = wave * 2 + ((lane >> 3) & 1);
    const float4 *xrow = xs + t * rs;
    const float4 *wrow = ws + j * rs;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        // pieces outside the quarter go to a junk slot: the stores stay
        // unconditional and the loads are not moved into a branch
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = lc + 32 * i;
            const uint4 v = xr[c][i];
            float4 *d = q < hq / 8 ? xs + lr * rs + (c * hq) / 4 + 2 * q : junk;
            d[0] = make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                               bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16));
            d[1] = make_float4(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16),
                               bf16_to_f32(v.w & 0xffffu), bf16_to_f32(v.w >> 16));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lc + 32 * i;
            float4 *d = q < hq / 4 ? ws + lr * rs + (c * hq) / 4 + q : junk;
            *d = wr[c][i];
        }
        __syncthreads();
        if (lane < 16) {
            const int b = (c * hq) / 4, n = hq / 4;     // float4 of this quarter
            float4 xa[4], wa[4], xb[4], wb[4];
            auto read = [&](int g, float4 (&xv)[4], float4 (&wv)[4]) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xv[i] = xrow[b + 4 * g + i];
                    wv[i] = wrow[b + 4 * g + i];
                }
            };
            auto fma16 = [&](const float4 (&xv)[4], const float4 (&wv)[4]) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = __builtin_fmaf(xv[i].x, wv[i].x, acc);
                    acc = __builtin_fmaf(xv[i].y, wv[i].y, acc);
                    acc = __builtin_fmaf(xv[i].z, wv[i].z, acc);
                    acc = __builtin_fmaf(xv[i].w, wv[i].w, acc);
                }
            };
            const int groups = n / 4;                   // even: hq is a multiple of 32
            read(0, xa, wa);
            for (int g = 0; g < groups; g += 2) {
                read(g + 1, xb, wb);
                __builtin_amdgcn_sched_barrier(0);
                fma16(xa, wa);
                __builtin_amdgcn_sched_barrier(0);
                read(g + 2 < groups ? g + 2 : g + 1, xa, wa);
                __builtin_amdgcn_sched_barrier(0);
                fma16(xb, wb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (lane < 16 && t < T && e0 + j < E)
        z[(size_t)t * E + e0 + j] = acc;
}

// LDS ints the fused plan of topk_block works in.
constexpr int kTopkLds = 2 * kFusedPlanMaxA + 2 * 256 + kMaxThreads / kWave;

// The top-k, the weights and (plan.counts given) the fused plan of the
// tokens of this workgroup, from z (global memory or LDS), with kTopkLds
// ints of LDS at lds. Every thread of the workgroup calls it.
template <int RE>
__device__ __forceinline__ void topk_block(const float *z, const float *__restrict__ bias, int T,
                                           int E, int k, int LPT, int norm_topk, float eps,
                                           int32_t *__restrict__ ids, float *__restrict__ weights,
                                           PlanOut plan, int *lds) {
    int *s_ids = lds;
    int *s_rank = s_ids + kFusedPlanMaxA;
    int *s_cnt = s_rank + kFusedPlanMaxA;
    int *s_off = s_cnt + 256;
    int *s_wsum = s_off + 256;
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
    // Assignment a's place within its expert is the number of earlier
    // assignments to the same expert, which keeps the scatter stable.
    __syncthreads();
    const int A = T * k;
    if (tid < E)
        s_cnt[tid] = 0;
    __syncthreads();
    for (int a = tid; a < A; a += kMaxThreads) {
        const int v = s_ids[a];
        int r = 0;
#pragma unroll 8
        for (int b = 0; b < a; ++b)
            r += s_ids[b] == v;
        s_rank[a] = r;
        atomicAdd(&s_cnt[v], 1);
    }
    __syncthreads();
    // exclusive scan of the counts: a wave scan per 64 experts
    int c = tid < E ? s_cnt[tid] : 0;
    int incl = c;
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += o;
    }
    if (lane == kWave - 1)
        s_wsum[tid / kWave] = incl;
    __syncthreads();
    for (int w = 0; w < tid / kWave; ++w)
        incl += s_wsum[w];
    if (tid < E) {
        s_off[tid] = incl - c;
        plan.counts[tid] = c;
        plan.offsets[tid] = incl - c;
        if (tid == E - 1)
            plan.offsets[E] = incl;
    }
    __syncthreads();
    for (int a = tid; a < A; a += kMaxThreads) {
        const int pos = s_off[s_ids[a]] + s_rank[a];
        plan.sorted[pos] = a;
        plan.slot_of[a] = pos;
    }
}

template <int RE>
__global__ __launch_bounds__(kMaxThreads) void k_topk(const float *__restrict__ z,
                                                      const float *__restrict__ bias, int T,
                                                      int E, int k, int LPT, int norm_topk,
                                                      float eps, int32_t *__restrict__ ids,
                                                      float *__restrict__ weights, PlanOut plan) {
    __shared__ int lds[kTopkLds];
    topk_block<RE>(z, bias, T, E, k, LPT, norm_topk, eps, ids, weights, plan, lds);
}

// k_route_decode: the whole router of a decode-sized batch (T <= 8,
// E <= 32, H a multiple of 128, H <= 2048) in one workgroup: the logits,
// then the top-k, the weights and the plan, with z kept in LDS. Lane l of
// wave w runs the chain of token l % 8 and expert 8 w + l / 8 (one chain per
// lane: the chain latency, H dependent fmas, is the floor of this step, so
// the loop carries nothing but the fmas and their LDS reads). The token
// rows are converted to fp32 into LDS once, at the start (rows padded by 16
// bytes: the 8 rows a read touches fall in distinct banks); the router rows
// stream through a ring of 5 LDS stages of 128 h, requested four stages
// ahead by range-checked buffer loads, pieces at swizzled slots (router row
// e: piece c ^ 2 (e % 8)).
constexpr int kDecT = 8;
constexpr int kDecE = 32;
constexpr int kDecMaxH = 2048;
constexpr int kDecXRow = kDecMaxH / 4 + 1;              // float4 per token row (+ pad)
constexpr int kDecX = kDecT * kDecXRow;                 // 65.6 KB
constexpr int kDecW = kDecE * (kRingH / 4);             // 1024 router pieces per stage (16 KB)
constexpr int kDecStages = 5;
constexpr int kDecAhead = kDecStages - 1;

// One stage: the chain over W's 128 h (x from X at float4 column c0), and the
// refill of stage F with h block sf. One call site, so the LDS reads and the
// loads into F share one alias scope.
__device__ __forceinline__ void dec_stage(const float4 *__restrict__ X,
                                          const uint4 *__restrict__ W, uint4 *__restrict__ F,
                                          const float *Wr, const uint32_t (&woff)[4], int sf,
                                          int c0, bool compute, float &acc) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        buffer_to_lds16(Wr, F + (q * 4 + wave) * kWave, woff[q] + sf * (kRingH * 4));
    if (!compute)
        return;
    const int t = lane & 7;
    const int e = wave * 8 + (lane >> 3);
    const float4 *xrow = X + t * kDecXRow + c0;
    const float4 *wrow = reinterpret_cast<const float4 *>(W) + e * (kRingH / 4);
    const int wsw = 2 * (e & 7);
    auto fma4 = [&](const float4 &xv, const float4 &wv) {
        acc = __builtin_fmaf(xv.x, wv.x, acc);
        acc = __builtin_fmaf(xv.y, wv.y, acc);
        acc = __builtin_fmaf(xv.z, wv.z, acc);
        acc = __builtin_fmaf(xv.w, wv.w, acc);
    };
    // 4 h per group; the reads run two groups ahead of the fmas
    constexpr int G = kRingH / 4;                           // 32 groups
    float4 xv[3], wv[3];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        xv[g] = xrow[g];
        wv[g] = wrow[g ^ wsw];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g + 2 < G) {
            xv[(g + 2) % 3] = xrow[g + 2];
            wv[(g + 2) % 3] = wrow[(g + 2) ^ wsw];
        }
        __builtin_amdgcn_sched_barrier(0);
        fma4(xv[g % 3], wv[g % 3]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(kMaxThreads) void k_route_decode(
    const uint16_t *__restrict__ x, const float *__restrict__ Wr, const float *__restrict__ bias,
    int T, int H, int E, int k, int LPT, int norm_topk, float eps, int32_t *__restrict__ ids,
    float *__restrict__ weights, PlanOut plan) {
    // one LDS object: the fp32 token rows, then the ring; reused after the
    // logits for z and the top-k's work space (a second LDS object would make
    // the compiler wait for every load into the ring before any read of it)
    __shared__ uint4 lds[kDecX + kDecStages * kDecW];   // 146 KB
    float4 *X = reinterpret_cast<float4 *>(lds);
    uint4 *ring = lds + kDecX;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int S = H / kRingH;
    // the token rows: 8 pieces of 8 bf16 per thread, in registers first,
    // by range-checked loads issued together (pieces past T or H read zeros)
    constexpr int kXPieces = kDecT * (kDecMaxH / 8) / kMaxThreads;
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, 0x7fffffff, kBufferWord3);
    uint4 xr[kXPieces];
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) {
        const int pos = i * kMaxThreads + tid;
        const int r = pos / (kDecMaxH / 8), c = pos % (kDecMaxH / 8);
        const uint32_t off = (r < T && 8 * c < H) ? ((uint32_t)r * (uint32_t)H + 8u * c) * 2u : kRingPast;
        xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, 0, 0));
    }
    // byte offsets of this thread's router pieces in h block 0; rows past E
    // read zeros
    uint32_t woff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int pos = (q * 4 + wave) * kWave + lane;
        const int j = pos / (kRingH / 4), c = (pos % (kRingH / 4)) ^ (2 * (j & 7));
        woff[q] = j < E ? ((uint32_t)j * (uint32_t)H + 4u * c) * 4u : kRingPast;
    }
    float acc = 0.0f;
    // Iterations -4 .. -1 only request h blocks 0 .. 3; every request comes
    // from the one call site below, in one alias scope. 4 requests per
    // iteration and wave (past the end the last h block again, into the
    // slot read in the previous iteration): stage s is in once at most the
    // 12 requests after it are in flight.
    for (int s = -kDecAhead; s < S; ++s) {
        wait_vmcnt<4 * (kDecAhead - 1)>();
        __builtin_amdgcn_s_barrier();       // also: the token rows are in LDS
        const int sc = s < 0 ? 0 : s;
        dec_stage(X, ring + (sc % kDecStages) * kDecW, ring + ((s + kDecAhead) % kDecStages) * kDecW,
                  Wr, woff, s + kDecAhead < S ? s + kDecAhead : S - 1, sc * (kRingH / 4), s >= 0,
                  acc);
        if (s == -1) {
            // the token rows to fp32, once the first router blocks are on
            // their way (visible after the next barrier)
#pragma unroll
            for (int i = 0; i < kXPieces; ++i) {
                const int pos = i * kMaxThreads + tid;
                const int r = pos / (kDecMaxH / 8), c = pos % (kDecMaxH / 8);
                const uint4 v = xr[i];
                float4 *d = X + r * kDecXRow + 2 * c;
                d[0] = make_float4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                                   bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16));
                d[1] = make_float4(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16),
                                   bf16_to_f32(v.w & 0xffffu), bf16_to_f32(v.w >> 16));
            }
        }
    }
    wait_vmcnt<0>();                        // the last requests land before the LDS is reused
    __syncthreads();                        // and every wave is past its reads
    float *zs = reinterpret_cast<float *>(lds);
    {
        const int t = lane & 7;
        const int e = wave * 8 + (lane >> 3);
        if (t < T && e < E)
            zs[t * E + e] = acc;
    }
    __syncthreads();
    topk_block<1>(zs, bias, T, E, k, LPT, norm_topk, eps, ids, weights, plan,
                  reinterpret_cast<int *>(lds) + kDecT * kDecE);
}

// Two chains per lane when that still leaves a few hundred workgroups,
// else one (decode-sized batches are latency-bound: more workgroups).
template <int C>
void launch_logits(hipStream_t stream, const uint16_t *x, const float *Wr, int T, int H, int E,
                   float *z) {
    const dim3 grid((T + kTok - 1) / kTok, (E + 4 * C - 1) / (4 * C));
    hipLaunchKernelGGL(k_logits<C>, grid, dim3(kMaxThreads), 0, stream, x, Wr, T, H, E, z);
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
    if (H % 64 != 0)
        return hipErrorInvalidValue;
    if (T <= kDecT && E <= kDecE && H % kRingH == 0 && H <= kDecMaxH) {
        // one workgroup: logits, top-k, weights and (when it fits) the plan
        int LPT = 2;
        while (LPT < E)
            LPT <<= 1;
        const bool fuse = plan.counts != nullptr && T * k <= kFusedPlanMaxA;
        if (!fuse)
            plan = PlanOut{};
        hipLaunchKernelGGL(k_route_decode, dim3(1), dim3(kMaxThreads), 0, stream, x, Wr, bias, T, H,
                           E, k, LPT, norm_topk, eps, ids, weights, plan);
        const hipError_t err = hipGetLastError();
        if (err == hipSuccess && plan_done != nullptr)
            *plan_done = fuse;
        return err;
    }
    const int tblocks = (T + kTok - 1) / kTok;
    if (T <= kFewT && H <= kFewMaxH && H % 128 == 0)
        hipLaunchKernelGGL(k_logits_few, dim3((E + kFewE - 1) / kFewE), dim3(kMaxThreads), 0,
                           stream, x, Wr, T, H, E, z_scratch);
    else if ((int64_t)tblocks * ((E + 7) / 8) >= 128 && H % kRingH == 0)
        hipLaunchKernelGGL(k_logits_ring, dim3(tblocks, (E + 7) / 8), dim3(kMaxThreads), 0, stream,
                           x, Wr, T, H, E, z_scratch);
    else if ((int64_t)tblocks * ((E + 7) / 8) >= 128)
        launch_logits<2>(stream, x, Wr, T, H, E, z_scratch);
    else
        launch_logits<1>(stream, x, Wr, T, H, E, z_scratch);
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
