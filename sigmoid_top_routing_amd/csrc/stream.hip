// stream.hip -- the decode form of the grouped expert GEMMs: each touched
// expert's weight rows are streamed from HBM once per call, against the few
// rows of its segment (TensorFold issue #548: decode rows and prompt rows
// take different kernels over the same weights; TileGym PR #187,
// "Performance": at batch 1 the block is bound by the weight bytes).
//
// Same problem as the MFMA GEMM (GemmProblem, same epilogues, same outputs),
// different shape of work, laid out for HBM throughput. A plain read of cold
// rows reaches about 6 TB/s on this part when each wave reads a few rows and
// the waves in flight cover one contiguous stretch of memory; it falls
// towards 4.5 TB/s when each wave walks dozens of rows, and further when the
// reads in flight are spread over many experts whose weights sit a multiple
// of 2 MB apart. So a wave here owns a single output unit (a gate/up row
// pair for SwiGLU, else one weight row), a workgroup owns 8 consecutive
// units of one expert, and consecutive workgroups take consecutive units of
// the same expert. Each wave requests its weight rows first, with fully
// coalesced 16-byte loads (64 lanes cover 1 KB of a row per instruction),
// while the workgroup stages the segment's token rows, up to 4 at a time,
// in LDS. Lane l takes elements 512 j + 8 l .. + 7 of every row, for every
// j, and accumulates with v_dot2_f32_bf16 (two bf16 products per
// instruction, fp32 accumulate). The 64 lane-partial sums of all rows are
// reduced with a transposing butterfly, which needs far fewer shuffles than
// reducing each value on its own, and one lane per row applies the epilogue.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A weight piece: read once per call, so the load is marked non-temporal
// (streamed past the caches rather than kept in them).
__device__ __forceinline__ uint4 stream_load(const uint16_t *p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}

constexpr int kThreads = 512;
constexpr int kTG = 4;         // token rows per group

// output units per wave: one (many short-lived waves stream fastest)
template <int NJ>
constexpr int units_per_wave() { return 1; }
template <int NJ>
constexpr int units_per_block() { return kThreads / kWave * units_per_wave<NJ>(); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &x, float c) {
    c = dot2(w.x, x.x, c);
    c = dot2(w.y, x.y, c);
    c = dot2(w.z, x.z, c);
    c = dot2(w.w, x.w, c);
    return c;
}

// v[0..V-1] hold lane partials of V sums. Halve the array log2(V/KEEP)
// times across lanes (xor 32, 16, ...), then sum the KEEP survivors over the
// remaining lanes. Afterwards v[0..KEEP-1] of every lane are full sums of
// the values whose index is given by the lane's bits 5, 4, ... (most
// significant first) times KEEP. Written as compile-time recursion, so every
// array index and xor mask is a constant (a runtime half would turn each
// v[j + half] into a chain of compares and selects).
template <int C, int KEEP, int M, int V>
__device__ __forceinline__ void transpose_reduce_step(float (&v)[V], int lane) {
    if constexpr (C > KEEP) {
        constexpr int half = C / 2;
        const bool hi = (lane & M) != 0;
#pragma unroll
        for (int j = 0; j < half; ++j) {
            const float give = hi ? v[j] : v[j + half];
            const float keep = hi ? v[j + half] : v[j];
            v[j] = keep + __shfl_xor(give, M, kWave);
        }
        transpose_reduce_step<half, KEEP, M / 2, V>(v, lane);
    } else if constexpr (M >= 1) {
#pragma unroll
        for (int j = 0; j < KEEP; ++j)
            v[j] += __shfl_xor(v[j], M, kWave);
        transpose_reduce_step<C, KEEP, M / 2, V>(v, lane);
    }
}

template <int V, int KEEP>
__device__ __forceinline__ void transpose_reduce(float (&v)[V], int lane) {
    transpose_reduce_step<V, KEEP, 32, V>(v, lane);
}

template <int MODE, int NJ>
__global__ __launch_bounds__(kThreads) void k_stream(GemmProblem p) {
    constexpr int NR = gated(MODE) ? 2 : 1;   // weight rows per unit
    constexpr int UW = units_per_wave<NJ>();
    __shared__ uint4 xs[kTG][NJ * kWave];          // token rows, bf16
    const int lane = threadIdx.x & (kWave - 1);
    // blockIdx.y names the expert among those with rows (in expert order),
    // so the workgroups in flight stream neighbouring rows of one or two
    // experts and none is spent on an empty one
    // (the segment's bounds come from the lane that tested the expert, so
    // the weight requests wait for one round of loads, not three)
    int e = 0, seg0 = 0, seg1 = p.rows;
    if (p.offsets != nullptr) {
        e = -1;
        int want = blockIdx.y;
        for (int base = 0; base < p.E && e < 0; base += kWave) {
            const int x = base + lane;
            const int lo = x < p.E ? p.offsets[x] : 0;
            const int hi = x < p.E ? p.offsets[x + 1] : 0;
            const bool busy = hi > lo;
            const uint64_t m = __ballot(busy);
            const int below = __popcll(m & ((1ull << lane) - 1ull));
            const uint64_t hit = __ballot(busy && below == want);
            if (hit != 0) {
                const int src = __ffsll((unsigned long long)hit) - 1;
                e = base + src;
                seg0 = __shfl(lo, src, kWave);
                seg1 = __shfl(hi, src, kWave);
            }
            want -= __popcll(m);
        }
        e = __builtin_amdgcn_readfirstlane(e);
        if (e < 0)
            return;                                // uniform
        seg0 = __builtin_amdgcn_readfirstlane(seg0);
        seg1 = __builtin_amdgcn_readfirstlane(seg1);
    }
    if (seg0 >= seg1)
        return;                                    // uniform
    const int units = gated(MODE) ? p.I : p.N;
    const int wave = threadIdx.x / kWave;
    const int K = p.K;
    const uint16_t *B = (const uint16_t *)p.B + (size_t)e * p.N * K;
    const int ub = blockIdx.x * units_per_block<NJ>() + wave * UW;

    // this wave's weight rows, requested before anything else
    uint4 w[UW][NR][NJ];
#pragma unroll
    for (int i = 0; i < UW; ++i) {
        const int u = ub + i;
#pragma unroll
        for (int s = 0; s < NR; ++s) {
            const uint16_t *wp = B + (size_t)(s == 0 ? u : p.I + u) * K;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int kk = j * 512 + lane * 8;
                w[i][s][j] = (u < units && kk < K) ? stream_load(wp + kk)
                                                   : make_uint4(0, 0, 0, 0);
            }
        }
    }

    for (int g0 = seg0; g0 < seg1; g0 += kTG) {
        const int nr = min(kTG, seg1 - g0);
        if (g0 != seg0)
            __syncthreads();                       // the previous group is read
        for (int idx = threadIdx.x; idx < kTG * NJ * kWave; idx += kThreads) {
            const int r = idx / (NJ * kWave), c = idx % (NJ * kWave);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < nr && c * 8 < K) {
                const int pos = g0 + r;
                const int arow = p.gather ? p.gather[pos] / p.gather_div : pos;
                v = *reinterpret_cast<const uint4 *>(p.A + (size_t)arow * p.lda + c * 8);
            }
            xs[r][c] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < UW; ++i) {
            const int u = ub + i;
            // values ordered (row r, weight row s): index r * NR + s
            float v[kTG * NR];
#pragma unroll
            for (int r = 0; r < kTG; ++r)
#pragma unroll
                for (int s = 0; s < NR; ++s) {
                    float acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        acc = dot8(w[i][s][j], xs[r][j * kWave + lane], acc);
                    v[r * NR + s] = acc;
                }
            transpose_reduce<kTG * NR, NR>(v, lane);
            // lane bits 5, 4 name the row r whose sums this lane now holds
            const int r = ((lane >> 5) & 1) * 2 + ((lane >> 4) & 1);
            if ((lane & 15) == 0 && r < nr && u < units) {
                const int pos = g0 + r;
                if (gated(MODE)) {
                    ((uint16_t *)p.C)[(size_t)pos * p.ldc + u] =
                        (uint16_t)f32_to_bf16(swiglu<MODE == kGateUpLimit>(v[0], v[1], p.limit));
                } else if (MODE == kUpRelu2) {
                    ((uint16_t *)p.C)[(size_t)pos * p.ldc + u] =
                        (uint16_t)f32_to_bf16(relu_sq(v[0]));
                } else {
                    const int orow = p.scatter ? p.scatter[pos] : pos;
                    ((float *)p.C)[(size_t)orow * p.ldc + u] = v[0];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Quantized weights in the decode form: the codes are streamed at their
// stored width and decoded in registers, so a step reads each touched
// expert's bytes once (TensorFold PR #1492, "What": the MLX 4-bit affine
// experts with group 64; TensorFold issue #548: block-FP8 experts with one
// fp32 scale per 128 x 128 block, and one decode-row kernel per format).
//
// A lane loads 16 bytes of codes per row and step j: 32 weights of 4-bit
// codes (elements 32 l + 2048 j .. + 31, inside one group of 64), or 16
// FP8 weights (elements 16 l + 1024 j .. + 15, inside one 128-wide K block).
// So each lane partial has a single scale, applied in fp32 to the partial:
//   4-bit:  w = s q + b, and sum_c w_c x_c = s (A - 128 X) + b X with
//           A = sum_c (128 + q_c) x_c and X = sum_c x_c over the lane's 32
//           elements. 128 + q is a bf16 whose bits are 0x4300 | q, so the
//           codes become bf16 pairs with two integer ops and A is a chain of
//           v_dot2_f32_bf16, like the bf16 kernel; X comes from the same
//           x reads (a dot2 chain with 1.0 pairs), once per token row and
//           step for all of the wave's units.
//   FP8:    w = s v, and sum_c w_c x_c = s (sum_c v_c x_c): every E4M3 value
//           is a bf16 value, so v is converted exactly (two per
//           instruction) and the sum is a v_dot2_f32_bf16 chain.
//   NVFP4:  32 E2M1 codes per lane and step (16 bytes), two 16-wide groups
//           with an E4M3 scale each: w = s_g v G, and the lane adds
//           s_0 (sum over group 0 of v x) + s_1 (sum over group 1), v
//           converted exactly (v_cvt_scalef32_pk_bf16_fp4, two per
//           instruction); the expert's global scale G multiplies the
//           reduced sum.
//   MXFP4:  the same 32 codes per lane and step, one E8M0 scale 2^(b-127)
//           for all of them: w = s v, the lane partial times s.
// The lane partials are then reduced across the wave as in k_stream.
constexpr int kFmtAffine4 = 1;
constexpr int kFmtFp8 = 2;
constexpr int kFmtNvfp4 = 3;
constexpr int kFmtMxfp4 = 4;

template <int FMT>
struct QFmt {
    static constexpr int EPL = FMT == kFmtFp8 ? 16 : 32;       // weights per lane per step
    static constexpr int EPJ = EPL * kWave;                    // weights per wave per step
    static constexpr int CPL = EPL / 8;                        // 16-byte x chunks per lane
};

// LDS slot of x chunk c (8 bf16) of a staged row: lane l reads chunks
// CPL l + i; the low bits are XORed with bits 4.. of the chunk so the 16
// lanes of one ds_read_b128 pass hit 16 distinct 16-byte bank groups.
template <int CPL>
__device__ __forceinline__ int qslot(int c) {
    return CPL == 1 ? c : ((c & ~(CPL - 1)) | ((c & (CPL - 1)) ^ ((c >> 4) & (CPL - 1))));
}

// 4-bit codes of one word -> four bf16 pairs (128 + q): pair b holds nibbles
// 2b (low half) and 2b + 1 (high half). v_perm_b32 puts byte b of w (low
// nibble: code 2b) in byte 0 and byte b of w >> 4 (low nibble: code 2b + 1)
// in byte 2 (selectors 0..3 pick bytes of its second operand, 4..7 of its
// first, 12 gives 0x00); the mask keeps those two nibbles under 0x4300.
__device__ __forceinline__ void q4_pairs(uint32_t w, uint32_t (&pr)[4]) {
    const uint32_t hi = w >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t t = __builtin_amdgcn_perm(hi, w, 0x0C000C00u | ((4u + b) << 16) | b);
        pr[b] = (t & 0x000F000Fu) | 0x43004300u;
    }
}

// Units per wave: two, or one at four steps of codes (the registers hold
// every step's codes). Four and eight weight rows per wave measured the same
// and slower (fewer waves fit a CU).
template <int NJ, int NR>
constexpr int q_units_per_wave() { return NJ >= 4 ? 1 : 2; }

template <int MODE, int FMT, int NJ>
__global__ __launch_bounds__(kThreads) void k_stream_q(GemmProblem p) {
    using Q = QFmt<FMT>;
    constexpr int NR = gated(MODE) ? 2 : 1;       // weight rows per unit
    constexpr int UW = q_units_per_wave<NJ, NR>();   // units per wave
    constexpr int XC = NJ * Q::EPJ / 8;           // x chunks per staged row
    __shared__ uint4 xs[kTG][XC];                 // token rows, bf16, swizzled chunks
    const int lane = threadIdx.x & (kWave - 1);
    int e = 0, seg0 = 0, seg1 = p.rows;
    if (p.offsets != nullptr) {
        e = -1;
        int want = blockIdx.y;
        for (int base = 0; base < p.E && e < 0; base += kWave) {
            const int x = base + lane;
            const int lo = x < p.E ? p.offsets[x] : 0;
            const int hi = x < p.E ? p.offsets[x + 1] : 0;
            const bool busy = hi > lo;
            const uint64_t m = __ballot(busy);
            const int below = __popcll(m & ((1ull << lane) - 1ull));
            const uint64_t hit = __ballot(busy && below == want);
            if (hit != 0) {
                const int src = __ffsll((unsigned long long)hit) - 1;
                e = base + src;
                seg0 = __shfl(lo, src, kWave);
                seg1 = __shfl(hi, src, kWave);
            }
            want -= __popcll(m);
        }
        e = __builtin_amdgcn_readfirstlane(e);
        if (e < 0)
            return;                                // uniform
        seg0 = __builtin_amdgcn_readfirstlane(seg0);
        seg1 = __builtin_amdgcn_readfirstlane(seg1);
    }
    if (seg0 >= seg1)
        return;                                    // uniform
    const int units = gated(MODE) ? p.I : p.N;
    const int wave = threadIdx.x / kWave;
    const int K = p.K;
    const int ub = blockIdx.x * (kThreads / kWave) * UW + wave * UW;

    // this wave's code rows and the scale (and bias) of each lane partial,
    // requested before anything else
    uint4 w[UW][NR][NJ];
    float sc[UW][NR][NJ], bi[UW][NR][NJ];
    const size_t erow = (size_t)e * p.N;
#pragma unroll
    for (int i = 0; i < UW; ++i) {
        const int u = ub + i;
#pragma unroll
        for (int s = 0; s < NR; ++s) {
            const int n = s == 0 ? u : p.I + u;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int kk = j * Q::EPJ + lane * Q::EPL;     // first weight of the lane
                const bool in = u < units && kk < K;
                sc[i][s][j] = 0.0f;
                bi[i][s][j] = 0.0f;
                if (FMT == kFmtAffine4 || FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
                    const uint8_t *row = (const uint8_t *)p.B + (erow + n) * (size_t)(K / 2);
                    w[i][s][j] = in ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(row + kk / 2)))
                                    : make_uint4(0, 0, 0, 0);
                    if (in && FMT == kFmtAffine4) {
                        const size_t g = (erow + n) * (size_t)(K / 64) + kk / 64;
                        sc[i][s][j] = bf16_to_f32(p.Bscale[g]);
                        bi[i][s][j] = bf16_to_f32(p.Bbias[g]);
                    } else if (in && FMT == kFmtMxfp4) {
                        // the one E8M0 scale of the lane's 32 codes
                        sc[i][s][j] = e8m0_to_f32(
                            ((const uint8_t *)p.Bscale)[(erow + n) * (size_t)(K / 32) + kk / 32]);
                    } else if (in) {
                        // the E4M3 scales of the lane's two 16-wide groups
                        // (sc: group 0, bi: group 1)
                        const uint32_t two = *reinterpret_cast<const uint16_t *>(
                            (const uint8_t *)p.Bscale + (erow + n) * (size_t)(K / 16) + kk / 16);
                        const uint32_t pr = __builtin_bit_cast(
                            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(two, 1.0f, false));
                        sc[i][s][j] = bf16_to_f32(pr & 0xffffu);
                        bi[i][s][j] = bf16_to_f32(pr >> 16);
                    }
                } else {
                    const uint8_t *row = (const uint8_t *)p.B + (erow + n) * (size_t)K;
                    w[i][s][j] = in ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(row + kk)))
                                    : make_uint4(0, 0, 0, 0);
                    if (in)
                        sc[i][s][j] = reinterpret_cast<const float *>(p.Bscale)
                            [((size_t)e * (p.N / 128) + n / 128) * (size_t)(K / 128) + kk / 128];
                }
            }
        }
    }

    for (int g0 = seg0; g0 < seg1; g0 += kTG) {
        const int nr = min(kTG, seg1 - g0);
        if (g0 != seg0)
            __syncthreads();                       // the previous group is read
        for (int idx = threadIdx.x; idx < kTG * XC; idx += kThreads) {
            const int r = idx / XC, c = idx % XC;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < nr && c * 8 < K) {
                const int pos = g0 + r;
                const int arow = p.gather ? p.gather[pos] / p.gather_div : pos;
                v = *reinterpret_cast<const uint4 *>(p.A + (size_t)arow * p.lda + c * 8);
            }
            xs[r][qslot<Q::CPL>(c)] = v;
        }
        __syncthreads();
        // v[i][r * NR + s]: unit i, token row r, weight row s
        float v[UW][kTG * NR];
#pragma unroll
        for (int i = 0; i < UW; ++i)
#pragma unroll
            for (int q = 0; q < kTG * NR; ++q)
                v[i][q] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            // step j of every unit's rows decoded to bf16 pairs once
            uint32_t pr[UW][NR][Q::EPL / 2];
#pragma unroll
            for (int i = 0; i < UW; ++i)
#pragma unroll
                for (int s = 0; s < NR; ++s) {
                    const uint32_t cw[4] = {w[i][s][j].x, w[i][s][j].y, w[i][s][j].z,
                                            w[i][s][j].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (FMT == kFmtAffine4) {
                            uint32_t four[4];
                            q4_pairs(cw[q], four);
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                pr[i][s][4 * q + b] = four[b];
                        } else if constexpr (FMT == kFmtNvfp4 || FMT == kFmtMxfp4) {
                            // byte b: codes 2b (low nibble) and 2b + 1
                            uint32_t four[4];
                            fp4_pairs(cw[q], four);
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                pr[i][s][4 * q + b] = four[b];
                        } else {
                            pr[i][s][2 * q] = __builtin_bit_cast(
                                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, false));
                            pr[i][s][2 * q + 1] = __builtin_bit_cast(
                                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, true));
                        }
                    }
                }
#pragma unroll
            for (int r = 0; r < kTG; ++r) {
                if (r < nr) {                      // uniform
                    // the lane's x values of this step, read once for every unit
                    uint4 xv[Q::CPL];
#pragma unroll
                    for (int c = 0; c < Q::CPL; ++c)
                        xv[c] = xs[r][qslot<Q::CPL>((j * kWave + lane) * Q::CPL + c)];
                    // 4-bit: X = the sum of those x values
                    float X = 0.0f;
                    if constexpr (FMT == kFmtAffine4) {
#pragma unroll
                        for (int c = 0; c < Q::CPL; ++c)
                            X = dot8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                0x3F803F80u), xv[c], X);
                    }
#pragma unroll
                    for (int i = 0; i < UW; ++i)
#pragma unroll
                        for (int s = 0; s < NR; ++s) {
                            if constexpr (FMT == kFmtNvfp4) {
                                // chunks 0, 1: group 0; chunks 2, 3: group 1
                                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                                for (int c = 0; c < 2; ++c)
                                    a0 = dot8(make_uint4(pr[i][s][4 * c], pr[i][s][4 * c + 1],
                                                         pr[i][s][4 * c + 2], pr[i][s][4 * c + 3]),
                                              xv[c], a0);
#pragma unroll
                                for (int c = 2; c < 4; ++c)
                                    a1 = dot8(make_uint4(pr[i][s][4 * c], pr[i][s][4 * c + 1],
                                                         pr[i][s][4 * c + 2], pr[i][s][4 * c + 3]),
                                              xv[c], a1);
                                v[i][r * NR + s] += sc[i][s][j] * a0;
                                v[i][r * NR + s] += bi[i][s][j] * a1;
                                continue;
                            }
                            float a = 0.0f;
#pragma unroll
                            for (int c = 0; c < Q::CPL; ++c)
                                a = dot8(make_uint4(pr[i][s][4 * c], pr[i][s][4 * c + 1],
                                                    pr[i][s][4 * c + 2], pr[i][s][4 * c + 3]),
                                         xv[c], a);
                            if constexpr (FMT == kFmtAffine4)
                                v[i][r * NR + s] += sc[i][s][j] * __builtin_fmaf(-128.0f, X, a) +
                                                    bi[i][s][j] * X;
                            else
                                v[i][r * NR + s] += sc[i][s][j] * a;
                        }
                }
            }
        }
        // the expert's global scale of the sums (NVFP4), uniform
        const float G = (FMT == kFmtNvfp4 && p.Bglobal != nullptr) ? p.Bglobal[e] : 1.0f;
#pragma unroll
        for (int i = 0; i < UW; ++i) {
            const int u = ub + i;
            transpose_reduce<kTG * NR, NR>(v[i], lane);
            if constexpr (FMT == kFmtNvfp4) {
#pragma unroll
                for (int q = 0; q < NR; ++q)
                    v[i][q] *= G;
            }
            const int r = ((lane >> 5) & 1) * 2 + ((lane >> 4) & 1);
            if ((lane & 15) == 0 && r < nr && u < units) {
                const int pos = g0 + r;
                if (gated(MODE)) {
                    ((uint16_t *)p.C)[(size_t)pos * p.ldc + u] = (uint16_t)f32_to_bf16(
                        swiglu<MODE == kGateUpLimit>(v[i][0], v[i][1], p.limit));
                } else if (MODE == kUpRelu2) {
                    ((uint16_t *)p.C)[(size_t)pos * p.ldc + u] =
                        (uint16_t)f32_to_bf16(relu_sq(v[i][0]));
                } else {
                    const int orow = p.scatter ? p.scatter[pos] : pos;
                    ((float *)p.C)[(size_t)orow * p.ldc + u] = v[i][0];
                }
            }
        }
    }
}

template <int MODE, int FMT, int NJ>
hipError_t launch_q(const GemmProblem &p, hipStream_t stream) {
    const int units = gated(MODE) ? p.I : p.N;
    const int upb = (kThreads / kWave) * q_units_per_wave<NJ, gated(MODE) ? 2 : 1>();
    const dim3 grid((units + upb - 1) / upb, p.offsets != nullptr ? p.E : 1);
    hipLaunchKernelGGL((k_stream_q<MODE, FMT, NJ>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int MODE, int FMT>
hipError_t launch_q_mode(const GemmProblem &p, hipStream_t stream) {
    const int nj = (p.K + QFmt<FMT>::EPJ - 1) / QFmt<FMT>::EPJ;
    if (nj <= 1)
        return launch_q<MODE, FMT, 1>(p, stream);
    if (nj <= 2)
        return launch_q<MODE, FMT, 2>(p, stream);
    return launch_q<MODE, FMT, 4>(p, stream);
}

template <int FMT>
hipError_t launch_q_fmt(const GemmProblem &p, hipStream_t stream) {
    switch (p.mode) {
    case kGateUp: return launch_q_mode<kGateUp, FMT>(p, stream);
    case kGateUpLimit: return launch_q_mode<kGateUpLimit, FMT>(p, stream);
    case kUpRelu2: return launch_q_mode<kUpRelu2, FMT>(p, stream);
    default: return launch_q_mode<kDown, FMT>(p, stream);
    }
}

// ---------------------------------------------------------------------------
// The decode form's down projection and the weighted combine in one launch.
// A workgroup owns 8 output columns for every expert with rows: it stages
// all the plan's rows (at most kDcRows of them, bf16) in LDS once; wave w
// takes column w % 8 and every second expert (from w / 8), streams that
// column's weight row of each of its experts in turn, and forms the expert's
// y values exactly as k_stream does (the same lane partials and butterfly);
// the y values stay in LDS. A wave has one weight row in flight at a time:
// the rows in flight then come from few experts at once, and with more of
// them ahead (two, four, six) the step took 0.6, 2.8 and 24 us longer, the
// reads spread over more experts' weights. Then the workgroup
// writes out[t, its columns] for every token exactly as k_combine does: acc =
// fma(w[t,j], y, acc) over j ascending from +0, times the routed scale (or
// the scale folded into each weight), plus the shared rows added in order,
// one rounding. No y leaves the workgroup and no second launch follows.
constexpr int kDcThreads = 1024;
constexpr int kDcCols = 8;          // output columns per workgroup
constexpr int kDcGroups = kDcThreads / kWave / kDcCols;   // waves per column
constexpr int kDcRows = 32;         // plan positions one launch takes
constexpr int kDcAhead = 1;         // experts whose weight rows a wave has in flight
constexpr int kDcMaxE = 256;

template <int NJ>
__global__ __launch_bounds__(kDcThreads) void k_down_combine(GemmProblem p, CombineArgs c) {
    __shared__ uint4 xs[kDcRows][NJ * kWave];       // the plan's rows, bf16
    __shared__ float ys[kDcRows][kDcCols];          // y[position][column]
    __shared__ int s_e[kDcMaxE], s_lo[kDcMaxE], s_hi[kDcMaxE];
    __shared__ int s_nb;
    __shared__ int s_slot[kDcRows];                 // the combine's inputs, loaded first
    __shared__ float s_w[kDcRows];
    __shared__ float s_sh[kDcRows][kDcCols];        // the shared rows' sum, per token
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int col = wave % kDcCols, grp = wave / kDcCols;
    // the combine's inputs (wave 1; wave 0 lists the experts): the slots, the
    // weights (the routed scale folded in with fold) and the shared rows
    // added in order, for this workgroup's columns
    if (wave == 1) {
        const int A = c.T * c.k;
        if (lane < A) {
            s_slot[lane] = c.slot[lane];
            s_w[lane] = c.fold ? c.rsf * c.w[lane] : c.w[lane];
        }
        for (int idx = lane; idx < c.T * kDcCols; idx += kWave) {
            const int t = idx / kDcCols, h = blockIdx.x * kDcCols + idx % kDcCols;
            float sh = 0.0f;
            if (c.shared != nullptr && h < p.N) {
                for (int v = 0; v < c.shared_terms; ++v) {
                    const float e = c.shared[((size_t)v * c.T + t) * p.N + h];
                    sh = v == 0 ? e : sh + e;
                }
            }
            s_sh[t][idx % kDcCols] = sh;
        }
    }
    const int K = p.K, N = p.N;
    const int u = blockIdx.x * kDcCols + col;       // this wave's output column
    // the experts with rows, in expert order
    if (wave == 0) {
        int nb = 0;
        for (int base = 0; base < p.E; base += kWave) {
            const int x = base + lane;
            const int lo = x < p.E ? p.offsets[x] : 0;
            const int hi = x < p.E ? p.offsets[x + 1] : 0;
            const bool busy = hi > lo;
            const uint64_t m = __ballot(busy);
            if (busy) {
                const int i = nb + __popcll(m & ((1ull << lane) - 1ull));
                s_e[i] = x;
                s_lo[i] = lo;
                s_hi[i] = hi;
            }
            nb += __popcll(m);
        }
        if (lane == 0)
            s_nb = nb;
    }
    __syncthreads();
    const int nb = s_nb;
    // this wave's weight row of its ii-th expert, busy expert grp + ii
    // kDcGroups (zeros past the list)
    auto load_row = [&](int ii, uint4 (&w)[NJ]) {
        const int i = grp + ii * kDcGroups;
        const bool ok = i < nb && u < N;
        const int e = ok ? s_e[i] : 0;
        const uint16_t *wp = (const uint16_t *)p.B + ((size_t)e * N + u) * K;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int kk = j * 512 + lane * 8;
            w[j] = (ok && kk < K) ? stream_load(wp + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 wb[kDcAhead][NJ];
#pragma unroll
    for (int q = 0; q < kDcAhead; ++q)
        load_row(q, wb[q]);
    // the plan's rows, while the first weight rows are in flight: every load
    // of a thread issued before its first LDS write
    const int A = p.offsets[p.E];
    constexpr int SL = kDcRows * NJ * kWave / kDcThreads;   // 16-byte pieces per thread
    uint4 sv[SL];
#pragma unroll
    for (int q = 0; q < SL; ++q) {
        const int idx = q * kDcThreads + threadIdx.x;
        const int r = idx / (NJ * kWave), cc = idx % (NJ * kWave);
        sv[q] = (r < A && cc * 8 < K)
                    ? *reinterpret_cast<const uint4 *>(p.A + (size_t)r * p.lda + cc * 8)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < SL; ++q) {
        const int idx = q * kDcThreads + threadIdx.x;
        xs[idx / (NJ * kWave)][idx % (NJ * kWave)] = sv[q];
    }
    __syncthreads();
    const int mine = nb > grp ? (nb - grp + kDcGroups - 1) / kDcGroups : 0;
    for (int i0 = 0; i0 < mine; i0 += kDcAhead) {
#pragma unroll
        for (int q = 0; q < kDcAhead; ++q) {
            const int ii = i0 + q;
            if (ii < mine) {                            // uniform
                const int i = grp + ii * kDcGroups;
                const int lo = s_lo[i], hi = s_hi[i];
                for (int g0 = lo; g0 < hi; g0 += kTG) {
                    const int nr = min(kTG, hi - g0);
                    float v[kTG];
#pragma unroll
                    for (int r = 0; r < kTG; ++r) {
                        float acc = 0.0f;
                        if (r < nr) {                   // uniform
#pragma unroll
                            for (int j = 0; j < NJ; ++j)
                                acc = dot8(wb[q][j], xs[g0 + r][j * kWave + lane], acc);
                        }
                        v[r] = acc;
                    }
                    transpose_reduce<kTG, 1>(v, lane);
                    // lane bits 5, 4 name the row r whose sum this lane now holds
                    const int r = ((lane >> 5) & 1) * 2 + ((lane >> 4) & 1);
                    if ((lane & 15) == 0 && r < nr)
                        ys[g0 + r][col] = v[0];
                }
            }
            load_row(ii + kDcAhead, wb[q]);
        }
    }
    __syncthreads();
    const int H = N;
    for (int idx = threadIdx.x; idx < c.T * kDcCols; idx += kDcThreads) {
        const int t = idx / kDcCols, cc = idx % kDcCols, h = blockIdx.x * kDcCols + cc;
        if (h >= H)
            continue;
        float acc = 0.0f;
        for (int j = 0; j < c.k; ++j)
            acc = __builtin_fmaf(s_w[t * c.k + j], ys[s_slot[t * c.k + j]][cc], acc);
        if (!c.fold)
            acc = acc * c.rsf;
        if (c.shared != nullptr)
            acc = acc + s_sh[t][cc];
        if (c.out_f32)
            ((float *)c.out)[(size_t)t * H + h] = acc;
        else
            ((uint16_t *)c.out)[(size_t)t * H + h] = (uint16_t)f32_to_bf16(acc);
    }
}

template <int MODE, int NJ>
hipError_t launch_nj(const GemmProblem &p, hipStream_t stream) {
    const int units = gated(MODE) ? p.I : p.N;
    const int upb = units_per_block<NJ>();
    const dim3 grid((units + upb - 1) / upb, p.offsets != nullptr ? p.E : 1);
    hipLaunchKernelGGL((k_stream<MODE, NJ>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const GemmProblem &p, hipStream_t stream) {
    const int nj = (p.K + 511) / 512;
    if (nj <= 1)
        return launch_nj<MODE, 1>(p, stream);
    if (nj <= 2)
        return launch_nj<MODE, 2>(p, stream);
    if (nj <= 4)
        return launch_nj<MODE, 4>(p, stream);
    return launch_nj<MODE, 8>(p, stream);
}

}  // namespace

bool stream_supported(const GemmProblem &p) {
    if (p.b_compact || p.scatter != nullptr || p.E2 > 0 || (p.Bglobal != nullptr && !p.nvfp4))
        return false;
    if (p.mxfp4)        // 4 code words per lane and step: one 32-wide block
        return p.K % 32 == 0 && p.K <= kStreamMaxKMxfp4;
    if (p.nvfp4)        // 4 code words per lane and step; groups of 16
        return p.K % 32 == 0 && p.K <= kStreamMaxKNvfp4;
    static_assert(kStreamMaxKAffine4 == 4 * QFmt<kFmtAffine4>::EPJ, "4-bit steps");
    static_assert(kStreamMaxKFp8 == 4 * QFmt<kFmtFp8>::EPJ, "FP8 steps");
    if (p.affine4)      // 4 code words per lane and step; groups of 64
        return p.K % 64 == 0 && p.K <= kStreamMaxKAffine4;
    if (p.fp8)          // 128 x 128 scale blocks
        return p.K % 128 == 0 && p.N % 128 == 0 && p.K <= kStreamMaxKFp8;
    return p.K <= 4096;
}

bool down_combine_supported(const GemmProblem &p, int T, int k) {
    return p.mode == kDown && !p.affine4 && !p.fp8 && !p.nvfp4 && !p.mxfp4 &&
           p.offsets != nullptr && p.E2 == 0 && p.scatter == nullptr && !p.b_compact &&
           p.Bglobal == nullptr && p.E <= kDcMaxE && p.K <= 2048 && p.N % 8 == 0 &&
           (int64_t)T * k <= kDcRows;
}

hipError_t launch_down_combine(const GemmProblem &p, const CombineArgs &c, hipStream_t stream) {
    if (!down_combine_supported(p, c.T, c.k))
        return hipErrorInvalidValue;
    const dim3 grid((p.N + kDcCols - 1) / kDcCols);
    const int nj = (p.K + 511) / 512;
    if (nj <= 1)
        hipLaunchKernelGGL(k_down_combine<1>, grid, dim3(kDcThreads), 0, stream, p, c);
    else if (nj <= 2)
        hipLaunchKernelGGL(k_down_combine<2>, grid, dim3(kDcThreads), 0, stream, p, c);
    else
        hipLaunchKernelGGL(k_down_combine<4>, grid, dim3(kDcThreads), 0, stream, p, c);
    return hipGetLastError();
}

hipError_t launch_stream(const GemmProblem &p, hipStream_t stream) {
    if (p.affine4)
        return launch_q_fmt<kFmtAffine4>(p, stream);
    if (p.fp8)
        return launch_q_fmt<kFmtFp8>(p, stream);
    if (p.nvfp4)
        return launch_q_fmt<kFmtNvfp4>(p, stream);
    if (p.mxfp4)
        return launch_q_fmt<kFmtMxfp4>(p, stream);
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp>(p, stream);
    case kGateUpLimit: return launch_mode<kGateUpLimit>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2>(p, stream);
    default: return launch_mode<kDown>(p, stream);
    }
}

}  // namespace moe
