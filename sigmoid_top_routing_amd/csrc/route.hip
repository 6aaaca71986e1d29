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
// order, and each (t, e)'s slices are added in order. k_logits_bc runs a
// lane per token, the router weights brought to the fmas by DPP from
// registers that hold 16 of them each; its byte offsets are formed from
// each workgroup's first token and router rows, so it takes any T and E
// (H <= 65536). Batches of at most 8 tokens and 32 experts take
// k_logits_part (the slices spread over the chip) and k_route_fold; at most
// 8 tokens with more experts, k_logits_few.
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

constexpr int kTok = 64;                 // tokens per workgroup (one per lane)

// k_logits_bc: a lane per token (64 tokens per workgroup) and CE experts
// (8 or 16) per workgroup; the eight waves share those tokens and experts and
// take alternate slices: in round m, wave w runs the CE chains of slice
// 8m + w.
// Eight waves (two per SIMD) because one wave alone cannot issue its fmas
// back to back. Each wave moves its own 64 token rows' 64 h for the next
// round (bf16) into its own two LDS stages by range-checked buffer loads,
// so it only ever waits on its own requests; a token row's 16-byte pieces
// (8 h) sit at piece c ^ (t / 2 mod 8) of its 128-byte LDS row, so 16 lanes
// reading their piece c hit 16 distinct 16-byte bank groups.
//
// The router weights go to registers, not LDS: lane l loads h 4(l mod 16) ..
// +3 of each of the CE router rows (the four 16-lane rows of the wave load
// the same 256 bytes), a round ahead, and the fma of h takes its weight from
// lane h / 4 of the lane's own 16-lane row through DPP (row_newbcast), so
// one register carries 16 weights of a slice. The chains themselves are
// unchanged: one v_fmac per term, h ascending from +0.
//
// After a round the eight slice partials go through LDS and wave w adds
// them, in slice order, to the running logits of experts e0 + w CE/8 ..
// +CE/8-1, which it writes at the end. A slice past the last one reads zeros, so its partial
// is +0, and adding +0 leaves a running sum that started at +0 unchanged (it
// is never -0): the fold has no branches.
constexpr int kBcWaves = 8;                           // waves per workgroup
constexpr int kBcThreads = kBcWaves * kWave;
constexpr int kBcStage = kTok * 8;                    // 16-byte x pieces per stage
constexpr uint32_t kBcPast = 0x80000000u;             // an offset that reads zeros

// acc = fma(w of lane N of this lane's 16-lane row, x, acc). A DPP
// instruction must not read a VGPR that a VALU instruction wrote in the two
// instructions before it; the callers keep every write of w, x and acc
// further away than that (w comes from global loads, x is converted a piece
// ahead, acc is written by the fma of the same chain CE instructions earlier
// or by the zeroing at the round's start).
template <int N>
__device__ __forceinline__ void fmac_bcast(float &acc, float w, float x) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc)
                 : "v"(w), "v"(x), "n"(N));
}

// the 8 h of a 16-byte piece of a bf16 row, as fp32
__device__ __forceinline__ void bc_convert(const uint4 v, float (&xs)[8]) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xs[2 * i] = __uint_as_float(u[i] << 16);
        xs[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

// the 8 CE fmas of piece P (h 8P .. 8P+7 of the slice), h ascending
template <int CE, int P>
__device__ __forceinline__ void bc_piece(float (&acc)[CE], const uint4 (&w)[CE],
                                         const float (&xs)[8]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 0; e < CE; ++e) {
                const uint32_t wj = j == 0 ? w[e].x : j == 1 ? w[e].y : j == 2 ? w[e].z : w[e].w;
                if (half == 0)
                    fmac_bcast<2 * P>(acc[e], __uint_as_float(wj), xs[j]);
                else
                    fmac_bcast<2 * P + 1>(acc[e], __uint_as_float(wj), xs[4 + j]);
            }
        }
    }
}

// One round of a wave. Request its next stage F (slice sn, zeros when fill
// is false) and that slice's router weights into wn; wait for this round's
// stage R + s_at and weights w; run the CE chains; exchange the partials
// through R + p_at and add the round's eight, in slice order, to z. Every
// LDS access but the requests goes through R: one alias scope for them and
// one for F, so the compiler neither orders the reads behind requests still
// in flight nor waits for those requests itself; the explicit wait does that.
template <int CE>
__device__ __forceinline__ void bc_round(uint4 *__restrict__ R, int s_at, int p_at,
                                         uint4 *__restrict__ F, const uint16_t *x,
                                         __amdgpu_buffer_rsrc_t wrsrc, const uint32_t (&xoff)[8],
                                         const uint32_t (&woff)[CE], int sn, bool fill,
                                         const uint4 (&w)[CE], uint4 (&wn)[CE],
                                         float (&z)[CE / kBcWaves]) {
    constexpr int Q = CE / kBcWaves;                    // experts this wave adds up
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
    for (int q = 0; q < 8; ++q)
        buffer_to_lds16(x, F + q * kWave, fill ? xoff[q] + (uint32_t)sn * 128u : kBcPast);
#pragma unroll
    for (int e = 0; e < CE; ++e)
        wn[e] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       wrsrc, fill ? woff[e] + (uint32_t)sn * 256u : kBcPast, 0, 0));
    // this round's stage and weights are in once only the 16 requests just
    // made may still be in flight
    wait_vmcnt<8 + CE>();
    __builtin_amdgcn_sched_barrier(0);
    const uint4 *S = R + s_at;
    uint4 xp[8];
    const int key = (lane >> 1) & 7;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        xp[c] = S[lane * 8 + (c ^ key)];
    // the chains start from +0 (a write the compiler cannot move next to
    // the first fma)
    float acc[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e)
        asm volatile("v_mov_b32 %0, 0" : "=v"(acc[e]));
    // each piece is converted while the fmas of the one before run
    float xa[8], xb[8];
    bc_convert(xp[0], xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[1], xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 0>(acc, w, xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[2], xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 1>(acc, w, xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[3], xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 2>(acc, w, xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[4], xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 3>(acc, w, xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[5], xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 4>(acc, w, xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[6], xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 5>(acc, w, xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_convert(xp[7], xb);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 6>(acc, w, xa);
    __builtin_amdgcn_sched_barrier(0);
    bc_piece<CE, 7>(acc, w, xb);
    __builtin_amdgcn_sched_barrier(0);
    // the exchange, [wave][expert][token] floats: every wave is done with
    // the last round's before any writes this round's
    float *P = reinterpret_cast<float *>(R + p_at);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < CE; ++e)
        P[(wave * CE + e) * kTok + lane] = acc[e];
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    float p[kBcWaves][Q];
#pragma unroll
    for (int v = 0; v < kBcWaves; ++v)
#pragma unroll
        for (int i = 0; i < Q; ++i)
            p[v][i] = P[(v * CE + wave * Q + i) * kTok + lane];
#pragma unroll
    for (int v = 0; v < kBcWaves; ++v)
#pragma unroll
        for (int i = 0; i < Q; ++i)
            z[i] = z[i] + p[v][i];
}

template <int CE>
__global__ __launch_bounds__(kBcThreads) void k_logits_bc(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ Wr, int T,
                                                          int H, int E, float *__restrict__ zout) {
    constexpr int RING = kBcWaves * 2 * kBcStage;       // two stages per wave
    constexpr int XCH = kBcWaves * CE * kTok / 4;        // the exchange, in 16-byte pieces
    constexpr int Q = CE / kBcWaves;                    // experts each wave adds up
    __shared__ uint4 lds[RING + XCH];                   // 144 KB (CE = 8) or 160 KB (16)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int t0 = blockIdx.x * kTok;
    const int e0 = blockIdx.y * CE;
    const int S = H / 64;
    const int M = (S + kBcWaves - 1) / kBcWaves;
    // byte offsets in slice 0 of this lane's requests, from the workgroup's
    // first token row and first router row (below 2^31 for H <= 65536, so
    // any T and E); rows past T or E read zeros
    const uint16_t *xw = x + (size_t)t0 * H;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(Wr + (size_t)e0 * H), (short)0, 0x7fffffff, kBufferWord3);
    uint32_t xoff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xoff[q] = t0 + r < T ? ((uint32_t)r * (uint32_t)H + 8u * c) * 2u : kBcPast;
    }
    uint32_t woff[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e)
        woff[e] = e0 + e < E ? ((uint32_t)e * (uint32_t)H + 4u * (lane & 15)) * 4u : kBcPast;
    const int mine = wave * (2 * kBcStage);
    // round 0's operands
    uint4 wa[CE], wb[CE];
    {
        const bool ok = wave < S;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            buffer_to_lds16(xw, lds + mine + q * kWave, ok ? xoff[q] + (uint32_t)wave * 128u : kBcPast);
#pragma unroll
        for (int e = 0; e < CE; ++e)
            wa[e] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           wrsrc, ok ? woff[e] + (uint32_t)wave * 256u : kBcPast, 0, 0));
    }
    float z[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i)
        z[i] = 0.0f;
    // two rounds per pass, so the weights alternate between wa and wb
    // without copies; both run (an odd last round reads zeros and adds +0),
    // as a load whose registers only a branch reads would be moved into it
    for (int m = 0; m < M; m += 2) {
        const int s1 = kBcWaves * (m + 1) + wave;
        bc_round<CE>(lds, mine, RING, lds + mine + kBcStage, xw, wrsrc, xoff, woff, s1, s1 < S, wa, wb,
                 z);
        const int s2 = kBcWaves * (m + 2) + wave;
        bc_round<CE>(lds, mine + kBcStage, RING, lds + mine, xw, wrsrc, xoff, woff, s2, s2 < S, wb, wa,
                 z);
    }
    // the requests of the round past the last (zeros) land before the
    // workgroup's LDS is given up
    wait_vmcnt<0>();
    const int t = t0 + lane;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int e = e0 + wave * Q + i;
        if (t < T && e < E)
            zout[(size_t)t * E + e] = z[i];
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
    else if (E >= 128)
        // 16 experts per workgroup: each token row is read by half as many
        // workgroups
        hipLaunchKernelGGL(k_logits_bc<16>, dim3(tblocks, (E + 15) / 16), dim3(kBcThreads), 0,
                           stream, x, Wr, T, H, E, z_scratch);
    else
        hipLaunchKernelGGL(k_logits_bc<8>, dim3(tblocks, (E + 7) / 8), dim3(kBcThreads), 0,
                           stream, x, Wr, T, H, E, z_scratch);
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
