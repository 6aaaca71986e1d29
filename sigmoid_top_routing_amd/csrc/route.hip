// route.hip -- router logits, sigmoid scores, bias-only top-k and weights.
//
// What is computed (TileGym PR #187, "Weight layout and routing"; TensorFold
// PR #1492, "What" and "Verification"):
//   p[t,e,j] = sum of x[t,h] * Wr[e,h] over slice j (h = 64 j .. 64 j + 63),
//              fp32, from +0, one fma per term, h ascending
//   z[t,e]   = p[t,e,0] + p[t,e,1] + ..., fp32, from +0, j ascending
//              (TensorFold issue #548: the router's K slices, fixed by H
//              alone, are added by the top-k; the width is not given, 64 is
//              this library's)
//   s[t,e]   = 1 / (1 + e^-z)           (own exp, correctly rounded division)
//              or, for the softmax router family (TensorFold issue #548, the
//              consolidation proposal): m = the row's largest non-NaN z,
//              q[e] = e^(z[e] - m) (0 below -87), S = q[0] + q[1] + ...
//              from +0 in expert order, s[t,e] = q[e] / S
//   key[t,e] = s[t,e] + bias[e]          (the bias only selects)
//   ids[t,:] = k experts by key, best first; ties to the lower index; NaN last
//   w[t,j]   = s[t,ids_j] / (sum_j s[t,ids_j] + eps)
//
// Two launches: the logits, then the top-k (which for decode-sized batches
// also adds the slices, k_route_fold).
//
// The logits are T*E*(H/64) independent fma chains of length 64, each in h
// order, and each (t, e)'s slices are added in order. k_logits_ring (H a
// multiple of 128) and k_logits (other H) run a lane per token; there the
// broadcast LDS reads of the router rows are what bound them. Batches of at
// most 8 tokens and 32 experts take k_logits_part (the slices spread over
// the chip) and k_route_fold; at most 8 tokens with more experts,
// k_logits_few.
//
// k_topk reads z, applies the sigmoid (or softmax) and the bias, and picks the top k of
// each token by the 64-bit (order key, ~index) candidates: with one expert
// per lane each lane counts the larger candidates of its token (its rank),
// else k rounds of xor-shuffle maxima over the token's lanes; then the
// weights. When one workgroup holds every token it also builds the plan.
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
// of the next 16 h are issued before the fmas of the current 16. Each slice
// of 64 h is one chain in h order, added to z when it ends.
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

    float acc[C], zc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        acc[c] = 0.0f;
        zc[c] = 0.0f;
    }
    // the slice just finished goes into z, and the next one starts at +0
    auto fold = [&]() {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            zc[c] = zc[c] + acc[c];
            acc[c] = 0.0f;
        }
    };
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
        const int groups = hc / 16;          // hc is a multiple of 64: 4 groups a slice
        read16(0, xa, wa);
        for (int g = 0; g < groups; g += 2) {
            read16(g + 1, xb, wb);
            __builtin_amdgcn_sched_barrier(0);
            fma16(xa, wa);
            __builtin_amdgcn_sched_barrier(0);
            read16(g + 2 < groups ? g + 2 : g + 1, xa, wa);   // no branch: no copies
            __builtin_amdgcn_sched_barrier(0);
            fma16(xb, wb);
            if ((g & 3) == 2)
                fold();
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
            z[(size_t)t * E + e] = zc[c];
    }
}

// k_logits_ring: the same lanes as k_logits<2> (a lane per token,
// two experts per wave: 64 tokens and 8 experts per workgroup), for H a
// multiple of 128. The operands come in by range-checked buffer loads
// straight into a ring of 4 LDS stages of 128 h (x as bf16, the router rows
// as fp32), requested three stages ahead, so the chains do not wait on
// memory once the ring is full; no registers hold staged data. A token row's
// 16-byte pieces (8 h) sit at piece c ^ (t % 16) of its LDS row, so the 16
// lanes of a 16-byte read hit distinct banks; the router rows are read by
// every lane at once (broadcast). A stage holds two slices.
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
    // The stage's two slices (h 0..63 and 64..127) run side by side: four
    // chains per lane (2 experts x 2 slices). 8 h per group and slice: one
    // 16-byte x piece, two float4 of each router row.
    auto read = [&](int g, uint4 (&xv)[2], float4 (&av)[2][2], float4 (&bv)[2][2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int q = g + 8 * j;
            xv[j] = xrow[q ^ (t & 15)];
            av[j][0] = wa[2 * q];
            av[j][1] = wa[2 * q + 1];
            bv[j][0] = wb[2 * q];
            bv[j][1] = wb[2 * q + 1];
        }
    };
    float pa[2] = {0.0f, 0.0f}, pb[2] = {0.0f, 0.0f};
    auto fma8 = [&](const uint4 (&xv)[2], const float4 (&av)[2][2], const float4 (&bv)[2][2]) {
        float xs[2][8], as[2][8], bs[2][8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 v = xv[j];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[j][2 * i] = bf16_to_f32(u[i] & 0xffffu);
                xs[j][2 * i + 1] = bf16_to_f32(u[i] >> 16);
            }
            const float4 a0 = av[j][0], a1 = av[j][1], b0 = bv[j][0], b1 = bv[j][1];
            const float al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float bl[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                as[j][i] = al[i];
                bs[j][i] = bl[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                pa[j] = __builtin_fmaf(xs[j][i], as[j][i], pa[j]);
                pb[j] = __builtin_fmaf(xs[j][i], bs[j][i], pb[j]);
            }
        }
    };
    uint4 xa[2], xb[2];
    float4 aa[2][2], ba[2][2], ab[2][2], bb[2][2];
    constexpr int G = kRingH / 16;                          // 8 groups per slice, even
    read(0, xa, aa, ba);
#pragma unroll
    for (int g = 0; g < G; g += 2) {
        read(g + 1, xb, ab, bb);
        __builtin_amdgcn_sched_barrier(0);
        fma8(xa, aa, ba);
        __builtin_amdgcn_sched_barrier(0);
        read(g + 2 < G ? g + 2 : G - 1, xa, aa, ba);       // no branch: no copies
        __builtin_amdgcn_sched_barrier(0);
        fma8(xb, ab, bb);
        __builtin_amdgcn_sched_barrier(0);
    }
    acc0 = acc0 + pa[0];
    acc0 = acc0 + pa[1];
    acc1 = acc1 + pb[0];
    acc1 = acc1 + pb[1];
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

// k_logits_few: at most 8 tokens with more than 32 experts (H <= 2048).
// The chains are the whole cost there (a lane runs its (t, e)'s slices one
// after another), so the point is to start them early and never stall
// them: a workgroup owns 8 experts and every
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
    float acc = 0.0f, zc = 0.0f;
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
            // a slice (64 h) ends after a group when the group's end is a
            // multiple of 64: its chain goes into z, the next starts at +0
            auto fold = [&](int g) {
                const bool end = ((c * hq + 16 * (g + 1)) & 63) == 0;
                zc = end ? zc + acc : zc;
                acc = end ? 0.0f : acc;
            };
            const int groups = n / 4;                   // even: hq is a multiple of 32
            read(0, xa, wa);
            for (int g = 0; g < groups; g += 2) {
                read(g + 1, xb, wb);
                __builtin_amdgcn_sched_barrier(0);
                fma16(xa, wa);
                fold(g);
                __builtin_amdgcn_sched_barrier(0);
                read(g + 2 < groups ? g + 2 : g + 1, xa, wa);
                __builtin_amdgcn_sched_barrier(0);
                fma16(xb, wb);
                fold(g + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (lane < 16 && t < T && e0 + j < E)
        z[(size_t)t * E + e0 + j] = zc;
}

// LDS ints the fused plan of topk_block works in.
constexpr int kTopkLds = 2 * kFusedPlanMaxA + 2 * 256 + kMaxThreads / kWave;

// The top-k, the weights and (plan.counts given) the fused plan of the
// tokens of this workgroup, from z (global memory or LDS), with kTopkLds
// ints of LDS at lds. Every thread of the workgroup calls it. RE experts
// per lane; with one, LPT <= MAXL.
template <int RE, int MAXL = 64>
__device__ __forceinline__ void topk_block(const float *z, const float *__restrict__ bias, int T,
                                           int E, int k, int LPT, int softmax, int norm_topk,
                                           float eps, int32_t *__restrict__ ids,
                                           float *__restrict__ weights, PlanOut plan, int *lds) {
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
    if (softmax) {
        // the row's largest non-NaN logit (exact: a max over the token's
        // lanes), the terms e^(z - m), and their sum in expert order: every
        // lane of the token adds the token's terms from LDS (the region of
        // the plan's ids, written again only after the barriers below)
        float zr[RE], q[RE];
        float m = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < RE; ++r) {
            const int e = eg + r * LPT;
            const bool real = t < T && e < E;
            zr[r] = real ? z[(size_t)t * E + e] : 0.0f;
            m = real && zr[r] > m ? zr[r] : m;
        }
        for (int msk = 1; msk < LPT; msk <<= 1) {
            const float o = __shfl_xor(m, msk, kWave);
            m = o > m ? o : m;
        }
        float *qs = reinterpret_cast<float *>(s_ids) + tb * LPT * RE;   // even: 8-byte aligned
#pragma unroll
        for (int r = 0; r < RE; ++r) {
            const int e = eg + r * LPT;
            q[r] = t < T && e < E ? softmax_term(zr[r] - m) : 0.0f;
            qs[e] = q[r];
        }
        __syncthreads();
        float S = 0.0f;
        for (int e = 0; e < E; e += 2) {
            const float2 v = *reinterpret_cast<const float2 *>(qs + e);
            S = S + v.x;
            S = e + 1 < E ? S + v.y : S;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RE; ++r)
            s[r] = q[r] / S;
    } else {
#pragma unroll
        for (int r = 0; r < RE; ++r) {
            const int e = eg + r * LPT;
            s[r] = t < T && e < E ? sigmoid_score(z[(size_t)t * E + e]) : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < RE; ++r) {
        const int e = eg + r * LPT;
        const bool real = t < T && e < E;
        s[r] = real ? s[r] : 0.0f;
        const float key = s[r] + (bias != nullptr && real ? bias[e] : 0.0f);
        cand[r] = real ? (((uint64_t)order_key(key) << 32) | (uint32_t)(0xffffu - e)) : 0ull;
    }
    if constexpr (RE == 1) {
        // One expert per lane: each lane ranks its candidate among its
        // token's (every lane of the token reads the token's LPT candidates
        // from LDS; the count of larger ones is the rank), and the lane of
        // rank j < k is pick j. No cross-lane shuffles on the way. The
        // candidates use the LDS of the plan's counts and offsets, the picked
        // scores that of its ranks: both are written again only after the
        // plan's first barrier.
        uint64_t *c64 = reinterpret_cast<uint64_t *>(s_cnt);
        float *pick_s = reinterpret_cast<float *>(s_rank);
        c64[tid] = cand[0];
        __syncthreads();
        const uint64_t *row = c64 + tb * LPT;
        int rank = 0;
#pragma unroll
        for (int i = 0; i < MAXL; i += 2) {
            // past LPT: a valid entry again, not counted (no branch)
            const ulonglong2 v = *reinterpret_cast<const ulonglong2 *>(row + (i & (LPT - 1)));
            rank += i < LPT ? (v.x > cand[0]) + (v.y > cand[0]) : 0;
        }
        const int e = eg;
        const bool pick = t < T && e < E && rank < k;
        if (pick) {
            ids[(size_t)t * k + rank] = e;
            pick_s[tb * k + rank] = s[0];
            if (plan.counts != nullptr)
                s_ids[tb * k + rank] = e;
        }
        __syncthreads();
        if (pick) {
            float sum = 0.0f;
            for (int j = 0; j < k; ++j)
                sum += pick_s[tb * k + j];
            const float denom = sum + eps;
            weights[(size_t)t * k + rank] = norm_topk ? s[0] / denom : s[0];
        }
    } else {
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
                                                      int E, int k, int LPT, int softmax,
                                                      int norm_topk, float eps,
                                                      int32_t *__restrict__ ids,
                                                      float *__restrict__ weights, PlanOut plan) {
    __shared__ __align__(16) int lds[kTopkLds];
    topk_block<RE>(z, bias, T, E, k, LPT, softmax, norm_topk, eps, ids, weights, plan, lds);
}

// The router of a decode-sized batch (T <= 8, E <= 32) in two launches.
// There are only T*E <= 256 logits, so one workgroup cannot keep many chains
// in flight, and every operand it reads from LDS feeds a single fma. The
// slices make the work split across the chip instead: k_logits_part gives
// each workgroup kPartSlices slices of every (t, e), loaded straight into
// registers (no LDS: lane l of wave w takes token l % 8 and expert
// 8 w + l / 8, and reads its own 256 bytes of router row and 128 bytes of
// token row per slice), and writes the partials p[j][t][e]. Then
// k_route_fold, one workgroup, adds each (t, e)'s partials in slice order
// into z (in LDS) and runs the top-k, the weights and the plan on it.
constexpr int kDecT = 8;
constexpr int kDecE = 32;
constexpr uint32_t kDecPast = 0x80000000u;             // an offset that reads zeros

// (one workgroup per CU: the registers go to the loads in flight). SP
// slices per workgroup.
template <int SP>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
k_logits_part(const uint16_t *__restrict__ x,
                                                             const float *__restrict__ Wr, int T,
                                                             int H, int E,
                                                             float *__restrict__ part) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int t = lane & 7;
    const int e = wave * 8 + (lane >> 3);
    const int S = H / 64;
    const int j0 = SP * blockIdx.x;
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, 0x7fffffff, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)Wr, (short)0, 0x7fffffff, kBufferWord3);
    // every load issued at once; rows past T or E and a slice past the end
    // read zeros
    uint4 xv[SP][8];
    float4 wv[SP][16];
#pragma unroll
    for (int j = 0; j < SP; ++j) {
        const int h0 = (j0 + j) * 64;
        const bool in = j0 + j < S;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off =
                (in && t < T) ? ((uint32_t)t * (uint32_t)H + (uint32_t)(h0 + 8 * i)) * 2u : kDecPast;
            xv[j][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t off =
                (in && e < E) ? ((uint32_t)e * (uint32_t)H + (uint32_t)(h0 + 4 * i)) * 4u : kDecPast;
            wv[j][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);                  // every request before any wait
    // the slices' chains side by side, h ascending in each
    float p[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j)
        p[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float xs[SP][8], ws[SP][8];
#pragma unroll
        for (int j = 0; j < SP; ++j) {
            const uint4 v = xv[j][i];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xs[j][2 * q] = bf16_to_f32(u[q] & 0xffffu);
                xs[j][2 * q + 1] = bf16_to_f32(u[q] >> 16);
            }
            const float4 a = wv[j][2 * i], b = wv[j][2 * i + 1];
            const float w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int q = 0; q < 8; ++q)
                ws[j][q] = w8[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
#pragma unroll
            for (int j = 0; j < SP; ++j)
                p[j] = __builtin_fmaf(xs[j][q], ws[j][q], p[j]);
        }
    }
    if (t < T && e < E) {
#pragma unroll
        for (int j = 0; j < SP; ++j)
            if (j0 + j < S)
                part[((size_t)(j0 + j) * T + t) * E + e] = p[j];
    }
}

constexpr int kPartSlices = 1;                          // slices per k_logits_part workgroup

constexpr int kFoldBatch = 32;                          // partial loads in flight per lane

__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
k_route_fold(
    const float *__restrict__ part, const float *__restrict__ bias, int T, int H, int E, int k,
    int LPT, int softmax, int norm_topk, float eps, int32_t *__restrict__ ids,
    float *__restrict__ weights, PlanOut plan) {
    __shared__ __align__(16) int lds[kDecT * kDecE + kDecE + kTopkLds];
    float *zs = reinterpret_cast<float *>(lds);
    float *bs = zs + kDecT * kDecE;                     // the bias, read with the partials
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int t = lane & 7;
    const int e = wave * 8 + (lane >> 3);
    const int S = H / 64;
    const bool real = t < T && e < E;
    const __amdgpu_buffer_rsrc_t prsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)part, (short)0, 0x7fffffff, kBufferWord3);
    const uint32_t base = real ? (uint32_t)(t * E + e) * 4u : kDecPast;
    const uint32_t stride = (uint32_t)(T * E) * 4u;
    const int tid = threadIdx.x;
    float b = 0.0f;
    if (bias != nullptr && tid < E)
        b = bias[tid];
    // z = ((+0 + p_0) + p_1) + ...: a batch of loads, then its adds in order
    float z = 0.0f;
    for (int j0 = 0; j0 < S; j0 += kFoldBatch) {
        float v[kFoldBatch];
#pragma unroll
        for (int i = 0; i < kFoldBatch; ++i) {
            const uint32_t off = j0 + i < S && real ? base + (uint32_t)(j0 + i) * stride : kDecPast;
            v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prsrc, off, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFoldBatch; ++i)
            z = j0 + i < S ? z + v[i] : z;
    }
    if (real)
        zs[t * E + e] = z;
    if (tid < E)
        bs[tid] = b;
    __syncthreads();
    topk_block<1, kDecE>(zs, bias != nullptr ? bs : nullptr, T, E, k, LPT, softmax, norm_topk,
                         eps, ids, weights, plan, lds + kDecT * kDecE + kDecE);
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

// Batches of at most 8 tokens and 32 experts take the two-launch decode
// router, whose scratch holds every slice's partial logits.
// (Its loads form 32-bit byte offsets into the router rows, E * H * 4 of
// them, which must stay below the buffer range of 2^31.)
bool decode_router(int T, int H, int E) {
    return T <= kDecT && E <= kDecE && (int64_t)E * H * 4 < ((int64_t)1 << 31);
}

size_t route_scratch_bytes(int T, int H, int E) {
    const size_t slices = decode_router(T, H, E) ? (size_t)(H / 64) : 1;
    return slices * T * E * sizeof(float);
}

hipError_t launch_route(const uint16_t *x, const float *Wr, const float *bias, int T, int H, int E,
                        int k, int softmax, int norm_topk, float eps, int32_t *ids,
                        float *weights, float *z_scratch, PlanOut plan, bool *plan_done,
                        hipStream_t stream) {
    if (plan_done != nullptr)
        *plan_done = false;
    if (T == 0)
        return hipSuccess;
    if (H % 64 != 0)
        return hipErrorInvalidValue;
    if (decode_router(T, H, E)) {
        // partial logits over the chip, then one workgroup: fold, top-k,
        // weights and (when it fits) the plan
        const int S = H / 64;
        hipLaunchKernelGGL(k_logits_part<kPartSlices>, dim3((S + kPartSlices - 1) / kPartSlices),
                           dim3(kMaxThreads), 0, stream, x, Wr, T, H, E, z_scratch);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        int LPT = 2;
        while (LPT < E)
            LPT <<= 1;
        const bool fuse = plan.counts != nullptr && T * k <= kFusedPlanMaxA;
        if (!fuse)
            plan = PlanOut{};
        hipLaunchKernelGGL(k_route_fold, dim3(1), dim3(kMaxThreads), 0, stream, z_scratch, bias, T,
                           H, E, k, LPT, softmax, norm_topk, eps, ids, weights, plan);
        err = hipGetLastError();
        if (err == hipSuccess && plan_done != nullptr)
            *plan_done = fuse;
        return err;
    }
    const int tblocks = (T + kTok - 1) / kTok;
    if (T <= kFewT && H <= kFewMaxH && H % 128 == 0)
        hipLaunchKernelGGL(k_logits_few, dim3((E + kFewE - 1) / kFewE), dim3(kMaxThreads), 0,
                           stream, x, Wr, T, H, E, z_scratch);
    else if ((int64_t)tblocks * ((E + 7) / 8) >= 128 && H % kRingH == 0 &&
             (int64_t)T * H * 2 < ((int64_t)1 << 31) && (int64_t)E * H * 4 < ((int64_t)1 << 31))
        // (the ring's requests form 32-bit byte offsets; an offset of 2^31
        // or more reads zeros)
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
                           k, LPT, softmax, norm_topk, eps, ids, weights, plan);
        break;
    case 2:
        hipLaunchKernelGGL(k_topk<2>, grid, dim3(kMaxThreads), 0, stream, z_scratch, bias, T, E,
                           k, LPT, softmax, norm_topk, eps, ids, weights, plan);
        break;
    default:
        hipLaunchKernelGGL(k_topk<4>, grid, dim3(kMaxThreads), 0, stream, z_scratch, bias, T, E,
                           k, LPT, softmax, norm_topk, eps, ids, weights, plan);
        break;
    }
    err = hipGetLastError();
    if (err == hipSuccess && plan_done != nullptr)
        *plan_done = fuse;
    return err;
}

}  // namespace moe
