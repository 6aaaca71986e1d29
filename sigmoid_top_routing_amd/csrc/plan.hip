// plan.hip -- the grouped expert plan: histogram, exclusive scan and a
// stable permutation of the assignments into per-expert segments
// (TensorFold issue #548: the routing plan shared by the grouped experts).
//
// Two launches. k_plan_count: each block counts the experts of one chunk of
// assignments into chunk_counts[chunk][E] with LDS atomics (integer sums, so
// the counts do not depend on their order). k_plan_scatter: each block sums
// the chunk counts column-wise, which gives every expert's total, the
// exclusive scan over experts (offsets) and the number of assignments of
// each expert in earlier chunks; it then walks its own chunk 256 assignments
// at a time. Inside a wave a lane's rank among lanes with the same expert
// comes from eight ballots (one per bit of the expert id); waves are ordered
// through a [wave][expert] count table in LDS. Positions therefore follow
// the assignment index inside every expert, with no order-dependent atomics.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 64;

// Also the shared segments (host-known, independent of the ids): the
// bounds after offsets[E] and the gather entries of their positions.
__global__ __launch_bounds__(kThreads) void k_plan_count(const int32_t *__restrict__ ids, int A,
                                                         int E, int chunk,
                                                         int32_t *__restrict__ chunk_counts,
                                                         int32_t *__restrict__ fault,
                                                         int32_t *__restrict__ sorted,
                                                         int32_t *__restrict__ seg_offsets,
                                                         int shared_segs, int T, int k) {
    if (shared_segs > 0) {
        const int n = shared_segs * T;
        for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
            sorted[A + i] = (i % T) * k;
        if (blockIdx.x == 0 && threadIdx.x < shared_segs)
            seg_offsets[E + 1 + threadIdx.x] = A + (threadIdx.x + 1) * T;
    }
    __shared__ int cnt[256];
    __shared__ int bad;
    const int tid = threadIdx.x;
    cnt[tid] = 0;
    if (tid == 0)
        bad = 0;
    __syncthreads();
    const int a0 = blockIdx.x * chunk;
    const int a1 = min(A, a0 + chunk);
    for (int a = a0 + tid; a < a1; a += kThreads) {
        const int e = ids[a];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            atomicAdd(&bad, 1);
    }
    __syncthreads();
    if (tid < E)
        chunk_counts[(size_t)blockIdx.x * E + tid] = cnt[tid];
    if (tid == 0 && bad > 0 && fault != nullptr)
        atomicAdd(fault, bad);
}

__global__ __launch_bounds__(kThreads) void k_plan_scatter(
    const int32_t *__restrict__ ids, int A, int E, int chunk, int nchunks,
    const int32_t *__restrict__ chunk_counts, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ slot_of,
    int32_t *__restrict__ seg_offsets) {
    __shared__ int run[256];
    __shared__ int wsum[4];
    __shared__ int wcnt[4][256];
    __shared__ int valid_total;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // totals, earlier-chunk counts and the exclusive scan over experts
    int total = 0, before = 0;
    if (tid < E) {
        // the loads of a batch are independent: one wait per 16 chunks
#pragma unroll 16
        for (int b = 0; b < nchunks; ++b) {
            const int c = chunk_counts[(size_t)b * E + tid];
            total += c;
            before += (b < (int)blockIdx.x) ? c : 0;
        }
    }
    int incl = total;
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += o;
    }
    if (lane == kWave - 1)
        wsum[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w)
        incl += wsum[w];
    const int excl = incl - total;
    if (tid == kThreads - 1)
        valid_total = incl;
    if (blockIdx.x == 0 && tid < E) {
        counts[tid] = total;
        offsets[tid] = excl;
        if (tid == E - 1)
            offsets[E] = incl;
        if (seg_offsets != nullptr) {
            seg_offsets[tid] = excl;
            if (tid == E - 1)
                seg_offsets[E] = incl;
        }
    }
    run[tid] = excl + before;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        wcnt[w][tid] = 0;
    __syncthreads();

    const int a0 = blockIdx.x * chunk;
    const int a1 = min(A, a0 + chunk);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int sub = a0; sub < a1; sub += kThreads) {
        const int a = sub + tid;
        const bool valid = a < a1;
        const int e = valid ? ids[a] : -1;
        const bool inr = valid && e >= 0 && e < E;
        uint64_t mask = __ballot(inr);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = inr && ((e >> bit) & 1);
            const uint64_t b = __ballot(on);
            mask &= on ? b : ~b;
        }
        const int rank = __popcll(mask & lt);
        if (inr && rank == 0)
            wcnt[wave][e] = __popcll(mask);
        __syncthreads();
        if (inr) {
            int pos = run[e] + rank;
            for (int w = 0; w < wave; ++w)
                pos += wcnt[w][e];
            sorted[pos] = a;
            slot_of[a] = pos;
        } else if (valid) {
            slot_of[a] = -1;
        }
        __syncthreads();
        run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            wcnt[w][tid] = 0;
        __syncthreads();
    }
    // positions no in-range assignment fills
    for (int p = a0 + tid; p < a1; p += kThreads)
        if (p >= valid_total)
            sorted[p] = -1;
}

}  // namespace

int plan_chunk_size(int A) {
    const int per = (A + kThreads * kMaxChunks - 1) / (kThreads * kMaxChunks);
    return kThreads * (per > 0 ? per : 1);
}

int plan_chunks(int A) {
    const int c = plan_chunk_size(A);
    return (A + c - 1) / c;
}

hipError_t launch_plan(const int32_t *ids, int A, int E, int32_t *counts, int32_t *offsets,
                       int32_t *sorted, int32_t *slot_of, int32_t *fault, int32_t *chunk_counts,
                       hipStream_t stream, int32_t *seg_offsets, int shared_segs, int T) {
    if (shared_segs < 0 || shared_segs > kThreads || (shared_segs > 0 && seg_offsets == nullptr) ||
        (shared_segs > 0 && (T <= 0 || A % T != 0)))
        return hipErrorInvalidValue;
    const int chunk = plan_chunk_size(A);
    const int nb = plan_chunks(A);
    if (nb > 0)
        hipLaunchKernelGGL(k_plan_count, dim3(nb), dim3(kThreads), 0, stream, ids, A, E, chunk,
                           chunk_counts, fault, sorted, seg_offsets, shared_segs, T,
                           shared_segs > 0 ? A / T : 0);
    // with no assignments one block still writes zero counts and offsets
    hipLaunchKernelGGL(k_plan_scatter, dim3(nb > 0 ? nb : 1), dim3(kThreads), 0, stream, ids, A,
                       E, chunk, nb, chunk_counts, counts, offsets, sorted, slot_of, seg_offsets);
    return hipGetLastError();
}

}  // namespace moe
