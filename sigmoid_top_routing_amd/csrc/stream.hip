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
// significant first) times KEEP.
template <int V, int KEEP>
__device__ __forceinline__ void transpose_reduce(float (&v)[V], int lane) {
    int c = V;
    int m = 32;
#pragma unroll
    for (int step = 0; (V >> step) > KEEP; ++step) {
        const bool hi = (lane & m) != 0;
        const int half = c / 2;
#pragma unroll
        for (int j = 0; j < V / 2; ++j) {
            if (j < half) {
                const float give = hi ? v[j] : v[j + half];
                const float keep = hi ? v[j + half] : v[j];
                v[j] = keep + __shfl_xor(give, m, kWave);
            }
        }
        c = half;
        m >>= 1;
    }
    for (; m >= 1; m >>= 1) {
#pragma unroll
        for (int j = 0; j < KEEP; ++j)
            v[j] += __shfl_xor(v[j], m, kWave);
    }
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
    return !p.affine4 && !p.fp8 && !p.b_compact && p.K <= 4096;
}

hipError_t launch_stream(const GemmProblem &p, hipStream_t stream) {
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp>(p, stream);
    case kGateUpLimit: return launch_mode<kGateUpLimit>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2>(p, stream);
    default: return launch_mode<kDown>(p, stream);
    }
}

}  // namespace moe
