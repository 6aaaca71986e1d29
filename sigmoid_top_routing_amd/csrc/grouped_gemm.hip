// grouped_gemm.hip -- persistent grouped expert GEMM for bf16 weights (gfx950).
//
// The same products as the staged kernel in gemm.hip,
//   C[p, n] = sum_k A[row(p), k] * B[e(p), n, k]   (fp32 accumulate),
// with the same fused epilogues (silu(g) * u for the gated up projection,
// relu^2 for the non-gated one, fp32 rows in segment order for the down
// projection; no output scatter), laid
// out for the matrix cores and the memory system of one MI355X:
//
// * Persistent workgroups. The grid is one workgroup per CU; each walks a
//   list of tiles (BM token rows of one expert x 256 weight rows), so a
//   tile's first operand slices are fetched while the previous tile is still
//   multiplying, and its output stores drain while the next one runs.
//
// * Tile order. Workgroups reach the 8 XCDs round robin (XCD = block % 8).
//   The real tiles are numbered expert by expert, and within an expert
//   n-tile major, m-tile minor; each XCD takes an equal contiguous share and
//   its 32 CUs sweep that share together. The tiles resident on an XCD at
//   one time are then all m-tiles of a run of n-tiles of one or two experts:
//   the m-tiles of a weight tile read it from HBM once and share it in that
//   XCD's L2, and the token rows of an m-tile are shared by its n-tiles.
//
// * Operands go from global memory straight into LDS (buffer loads with the
//   LDS bit, 16 bytes per lane) through a ring of 4 stages of K = 32,
//   requested 3 stages ahead of the one being multiplied. The request stream
//   runs across tile boundaries: the last steps of a tile request the first
//   slices of the next. No VGPRs hold staged data and no LDS writes are
//   issued by the waves. Each request's byte offset at K-slice 0 is formed
//   once per tile, so a step only adds the slice offset. Token rows past a
//   segment (padding of its last tile) are read as zeros by the range check,
//   which costs no memory traffic; weight rows past N are clamped to a valid
//   row. Neither result is stored.
//
// * The MFMA v_mfma_f32_32x32x16_bf16 is issued with the weight fragment as
//   its first operand, so the 32x32 accumulator tile is [weight row][token]:
//   each lane owns one token and, per group of 4 result registers, 4
//   consecutive output columns, which the epilogue packs (4 bf16 or 4 fp32)
//   and stores directly.
//
// * A step (K = 32) is two sub-steps of TM x TN independent MFMAs. Every LDS
//   read and every global request sits between two MFMAs (scheduling fences
//   keep the written order): sub-step 0 reads the fragments of sub-step 1;
//   then one barrier makes the next stage visible; sub-step 1 reads the next
//   step's first fragments and requests the stage 3 steps ahead.
//
// Ring hazards. The stage refilled in step g is the one read in step g - 1,
// whose last fragment reads were consumed by MFMAs before the barrier of
// step g, and the refill is requested after that barrier. A stage is read
// only after a barrier preceded by each wave's wait for its own requests of
// that stage (s_waitcnt vmcnt). The LDS reads and the refill of one step go
// through separate __restrict__ pointers, so the compiler does not order the
// reads behind the requests still in flight; the explicit waits do that.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;          // K per ring stage
// Ring depth: NS stages, NS - 1 requested ahead of the one multiplied. Four
// for 256-row tiles (32 KB stages); six for 128-row tiles (24 KB stages),
// which carry half the MFMAs per weight byte and stream weights from HBM
// when segments are short, so they need more bytes in flight.
constexpr int kStagesSmall = 4;
constexpr int kStagesDeep = 6;
constexpr int kBN = 256;         // weight rows per tile
constexpr int kXcds = 8;
constexpr int kMaxE = 256;
constexpr uint32_t kPastA = 0x80000000u;   // an A offset past every A matrix: reads zeros

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) volatile u32x4 lds_u32x4;

// 16-byte slot of logical chunk c (of 4 per row of 32 bf16) of row r within a
// stage. A fragment read serves 16 lanes (16 consecutive rows, one chunk) per
// pass from 64 banks; bits 0-1 of the row pick the 64-byte quarter of the
// 256-byte bank window and the chunk is XORed with bits 2-3 of the row.
__device__ __forceinline__ int slot_of(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// LDS accesses of the epilogue, each through a __restrict__ pointer: the
// compiler waits for every request still in flight into LDS before an LDS
// access it cannot place in an alias scope, and these give it one.
__device__ __forceinline__ void park_put16(char *__restrict__ base, int off, u32x4 v) {
    *(lds_u32x4 *)(base + off) = v;
}
__device__ __forceinline__ void park_put8(char *__restrict__ base, int off, u32x2 v) {
    *(__attribute__((address_space(3))) volatile u32x2 *)(base + off) = v;
}
__device__ __forceinline__ u32x4 park_get16(char *__restrict__ base, int off) {
    return (u32x4) * (lds_u32x4 *)(base + off);
}

template <int BM>
struct Geo {
    static constexpr int TM = BM / 64;            // 32-token MFMA tiles per wave
    static constexpr int TN = kBN / 64;           // 32-weight-row MFMA tiles per wave
    static constexpr int AI = BM * 4 / kThreads;  // A requests per thread per stage
    static constexpr int BI = kBN * 4 / kThreads; // B requests per thread per stage
    static constexpr int PER = AI + BI;
    static constexpr int STAGE = (BM + kBN) * 4;  // 16-byte slots per stage
    static constexpr int NQ = TM * TN;            // MFMAs per sub-step
    static constexpr int NF = TM + TN;            // fragment reads per sub-step
};

// Where the tiles of one launch are: the prefix of tiles over the segments
// (a dense problem is one segment) and this workgroup's share of the list.
struct TileList {
    const int *pre;      // LDS: first tile index of each segment
    const int *off;      // LDS: first row of each segment, and the end
    int nseg, n_tiles, work, share, xcd, cslot, nslots;
};

// Uniform placement of this workgroup's i-th tile; false past the end.
template <int BM>
__device__ __forceinline__ bool place(const TileList &tl, int i, int &e, int &row0, int &row_end,
                                      int &nt) {
    const int local = tl.cslot + i * tl.nslots;
    const int L = tl.xcd * tl.share + local;
    if (local >= tl.share || L >= tl.work)
        return false;
    // segment e owns tiles pre[e] * n_tiles .. pre[e + 1] * n_tiles - 1: the
    // last e with pre[e] <= L / n_tiles (empty segments share their prefix
    // with the next one and are skipped)
    const int mq = L / tl.n_tiles;
    int lo = 0, hi = tl.nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tl.pre[mid] <= mq)
            lo = mid;
        else
            hi = mid - 1;
    }
    // within the segment n-major, m-minor: the m-tiles that share a weight
    // tile are neighbours in the list, so they run at the same time on one
    // XCD and the weight rows are read from HBM once
    const int me = tl.pre[lo + 1] - tl.pre[lo];
    const int local_t = L - tl.pre[lo] * tl.n_tiles;
    e = __builtin_amdgcn_readfirstlane(lo);
    row0 = __builtin_amdgcn_readfirstlane(tl.off[lo] + (local_t % me) * BM);
    row_end = __builtin_amdgcn_readfirstlane(tl.off[lo + 1]);
    nt = __builtin_amdgcn_readfirstlane(local_t / me);
    return true;
}

// The A row behind each of this thread's A pieces of a tile, as stored in
// the plan (a slot, divided by gather_div once it has arrived). Returns a
// mask of the pieces that lie on rows of the segment; the others (rows past
// its end, which only pad the tile) are read as zeros.
template <int BM>
__device__ __forceinline__ int gathered_rows(const GemmProblem &p, int row0, int row_end,
                                             int (&raw)[Geo<BM>::AI]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int valid = 0;
#pragma unroll
    for (int i = 0; i < Geo<BM>::AI; ++i) {
        int pos = row0 + (((wave * Geo<BM>::AI + i) * kWave + lane) >> 2);
        valid |= (pos < row_end ? 1 : 0) << i;
        if (pos >= row_end)
            pos = row_end - 1;
        raw[i] = p.gather ? p.gather[pos] : pos;
    }
    return valid;
}

template <int BM>
__device__ __forceinline__ void a_offsets(const GemmProblem &p, const int (&raw)[Geo<BM>::AI],
                                          int valid, uint32_t (&off)[Geo<BM>::AI]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < Geo<BM>::AI; ++i) {
        const int s = (wave * Geo<BM>::AI + i) * kWave + lane;
        const int c = (s & 3) ^ ((s >> 4) & 3);
        const int arow = p.gather ? raw[i] / p.gather_div : raw[i];
        off[i] = (valid >> i) & 1 ? ((uint32_t)arow * (uint32_t)p.lda + c * 8) * 2u : kPastA;
    }
}

// Request state of the tile whose slices are being fetched.
template <int BM>
struct Req {
    const char *b_base;               // uniform: the expert's weight rows
    uint32_t a_off[Geo<BM>::AI];      // per thread, bytes at K-slice 0
    uint32_t b_off[Geo<BM>::BI];
};

// The weight side of a tile's requests: the expert's base and, per B piece
// of this thread, the byte offset of its row and chunk at K-slice 0 (rows
// past N are clamped to a valid row).
template <int BM, int MODE>
__device__ __forceinline__ void b_offsets(const GemmProblem &p, int e, int nt, Req<BM> &q) {
    using G = Geo<BM>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    q.b_base = (const char *)p.B + (size_t)e * p.N * p.K * 2;
#pragma unroll
    for (int i = 0; i < G::BI; ++i) {
        const int s = (wave * G::BI + i) * kWave + lane;
        const int r = s >> 2;
        const int c = (s & 3) ^ ((r >> 2) & 3);
        int wr;
        if (gated(MODE)) {
            int n = nt * (kBN / 2) + (r & (kBN / 2 - 1));
            if (n >= p.I)
                n = p.I - 1;
            wr = r < kBN / 2 ? n : p.I + n;
        } else {
            wr = nt * kBN + r;
            if (wr >= p.N)
                wr = p.N - 1;
        }
        q.b_off[i] = ((uint32_t)wr * (uint32_t)p.K + c * 8) * 2u;
    }
}

// Piece m (A pieces first, then B pieces) of K-slice ks into one stage.
template <int BM, int MODE>
__device__ __forceinline__ void request(uint4 *__restrict__ stage, const GemmProblem &p,
                                        const Req<BM> &q, int ks, int m) {
    using G = Geo<BM>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t kb = (uint32_t)ks * (kBK * 2);
    if (m < G::AI) {
        // pieces of padding rows (offset kPastA) read as zeros
        buffer_to_lds16(p.A, stage + (wave * G::AI + m) * kWave, q.a_off[m] + kb);
    } else {
        const int i = m - G::AI;
        buffer_to_lds16(q.b_base, stage + BM * 4 + (wave * G::BI + i) * kWave, q.b_off[i] + kb);
    }
}

// Fragment registers: slot 0 and 1 of a double buffer over sub-steps.
template <int BM>
struct Frags {
    bf16x8 a[2][Geo<BM>::TM];
    bf16x8 b[2][Geo<BM>::TN];
};

// Fragment m from a stage into a slot, in the order the MFMAs of a sub-step
// first use them (they run weight tile j fastest): A tile 0, B tiles 0 ..
// TN - 1, then A tiles 1 .. TM - 1. The reads of a sub-step are spread over
// its MFMAs, so the ones needed first by the next sub-step are in flight
// longest.
template <int BM>
__device__ __forceinline__ void read_frag(const uint4 *__restrict__ S, Frags<BM> &f, int slot, int m,
                                          int a_slot, int b_slot, const int *b_toff) {
    using G = Geo<BM>;
    if (m == 0)
        f.a[slot][0] = __builtin_bit_cast(bf16x8, S[a_slot]);
    else if (m <= G::TN)
        f.b[slot][m - 1] = __builtin_bit_cast(bf16x8, S[b_slot + b_toff[m - 1]]);
    else
        f.a[slot][m - G::TN] = __builtin_bit_cast(bf16x8, S[a_slot + (m - G::TN) * 128]);
}

// One step: multiply stage S (its sub-step 0 fragments are already in slot
// 0), read the next step's first fragments from Snext, refill Sfill with
// K-slice ks of the requested tile.
template <int BM, int MODE, int NS>
__device__ __forceinline__ void ring_step(const uint4 *__restrict__ S, const uint4 *__restrict__ Snext,
                                          uint4 *__restrict__ Sfill, const GemmProblem &p,
                                          const Req<BM> &q, int ks, Frags<BM> &f,
                                          f32x16 (&acc)[Geo<BM>::TM][Geo<BM>::TN],
                                          const int (&a_slot)[2], const int (&b_slot)[2],
                                          const int *b_toff) {
    using G = Geo<BM>;
    fence();
    // sub-step 0: MFMAs on slot 0, fragments of sub-step 1 into slot 1
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / G::TN, j = n % G::TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[0][j], f.a[0][i], acc[i][j], 0, 0, 0);
        // one read per MFMA from the first: all have landed by the
        // barrier, where the next sub-step starts
        if (n < G::NF)
            read_frag<BM>(S, f, 1, n, a_slot[1], b_slot[1], b_toff);
        fence();
    }
    // the next stage is complete once every wave's own requests for it are:
    // only the requests of the NS - 3 stages after it may still be in flight
    wait_vmcnt<(NS - 3) * G::PER>();
    __builtin_amdgcn_s_barrier();
    fence();
    // sub-step 1: MFMAs on slot 1, the next step's first fragments into
    // slot 0, and the refill of the stage read in the previous step
    constexpr int NM = G::NF + G::PER;
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / G::TN, j = n % G::TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[1][j], f.a[1][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int m = n * NM / G::NQ; m < (n + 1) * NM / G::NQ; ++m) {
            if (m < G::NF)
                read_frag<BM>(Snext, f, 0, m, a_slot[0], b_slot[0], b_toff);
            else
                request<BM, MODE>(Sfill, p, q, ks, m - G::NF);
        }
        fence();
    }
}

// Prologue: the first NS - 1 slices of the first tile into stages 0 ..
// NS - 2.
template <int BM, int MODE, int NS>
__device__ __forceinline__ void prime(uint4 *__restrict__ ring, const GemmProblem &p,
                                      const Req<BM> &q) {
    using G = Geo<BM>;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
#pragma unroll
        for (int m = 0; m < G::PER; ++m)
            request<BM, MODE>(ring + st * G::STAGE, p, q, st, m);
}

template <int BM, int MODE, int NS>
__global__ __launch_bounds__(kThreads, 1) void k_grouped(GemmProblem p, int n_tiles) {
    using G = Geo<BM>;
    constexpr int TM = G::TM, TN = G::TN;
    constexpr int kAhead = NS - 1;           // stages requested ahead of the one multiplied
    __shared__ uint4 ring[NS * G::STAGE];
    // the epilogue's wave-private 4 KB (256-row tiles; 128-row tiles use the
    // stage multiplied last). An LDS object of its own, so the compiler can
    // tell its reads from the requests still in flight into the ring.
    __shared__ uint4 park_lds[BM == 256 ? 4 * 256 : 1];
    __shared__ int s_pre[kMaxE + 1];
    __shared__ int s_off[kMaxE + 1];
    __shared__ int s_rank[kMaxE];            // compact B: a segment's place among those with rows
    __shared__ int s_wsum[4];
    __shared__ int s_bsum[4];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- tiles per segment and their prefix
    const int nseg = p.offsets ? p.E : 1;
    int tiles = 0;
    if (tid < nseg) {
        const int lo = p.offsets ? p.offsets[tid] : 0;
        const int hi = p.offsets ? p.offsets[tid + 1] : p.rows;
        s_off[tid] = lo;
        if (tid == nseg - 1)
            s_off[nseg] = hi;
        tiles = (hi - lo + BM - 1) / BM;
    }
    int incl = tiles;
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += o;
    }
    if (lane == kWave - 1)
        s_wsum[wave] = incl;
    const uint64_t busy = __ballot(tid < nseg && tiles > 0);
    if (lane == 0)
        s_bsum[wave] = __popcll(busy);
    __syncthreads();
    if (tid < nseg) {
        int rank = __popcll(busy & ((1ull << lane) - 1ull));
        for (int w = 0; w < wave; ++w)
            rank += s_bsum[w];
        s_rank[tid] = rank;
    }
    int total = 0;
    for (int w = 0; w < 4; ++w) {
        if (w < wave)
            incl += s_wsum[w];
        total += s_wsum[w];
    }
    if (tid < nseg)
        s_pre[tid] = incl - tiles;
    if (tid == 0)
        s_pre[nseg] = total;
    __syncthreads();

    // ---- this workgroup's tiles: an equal contiguous share per XCD, swept
    // by that XCD's workgroups in step
    TileList tl;
    tl.pre = s_pre;
    tl.off = s_off;
    tl.nseg = nseg;
    tl.n_tiles = n_tiles;
    tl.work = __builtin_amdgcn_readfirstlane(total) * n_tiles;
    tl.share = (tl.work + kXcds - 1) / kXcds;
    tl.xcd = blockIdx.x % kXcds;
    tl.cslot = blockIdx.x / kXcds;
    tl.nslots = gridDim.x / kXcds;

    int e, row0, row_end, nt;                // the tile being multiplied
    if (!place<BM>(tl, 0, e, row0, row_end, nt))
        return;                              // uniform
    Req<BM> req;                             // the tile being fetched
    {
        int raw[G::AI];
        const int valid = gathered_rows<BM>(p, row0, row_end, raw);
        a_offsets<BM>(p, raw, valid, req.a_off);
        b_offsets<BM, MODE>(p, p.b_compact ? s_rank[e] : e, nt, req);
    }
    int ne, nrow0, nrow_end, nnt;            // the next tile (if any)
    bool has_next = place<BM>(tl, 1, ne, nrow0, nrow_end, nnt);
    int nraw[G::AI];
    int nvalid = gathered_rows<BM>(p, has_next ? nrow0 : row0, has_next ? nrow_end : row_end, nraw);

    // LDS slots of this lane's fragment pieces for sub-steps 0 and 1; the
    // tiles of a wave sit 32 rows apart, which keeps the swizzle (+128 slots)
    const int a_tile_row = wm * (BM / 2);
    const int b_row0 = gated(MODE) ? wn * (kBN / 4) : wn * (kBN / 2);
    int b_toff[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (gated(MODE))
            b_toff[j] = ((j < TN / 2) ? j * 32 : kBN / 2 + (j - TN / 2) * 32) * 4;
        else
            b_toff[j] = j * 32 * 4;
    }
    int a_slot[2], b_slot[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        a_slot[kk] = slot_of(a_tile_row + (lane & 31), ch);
        b_slot[kk] = BM * 4 + slot_of(b_row0 + (lane & 31), ch);
    }

    const int KT = p.K / kBK;
    prime<BM, MODE, NS>(ring, p, req);
    wait_vmcnt<(NS - 2) * G::PER>();
    __builtin_amdgcn_s_barrier();
    Frags<BM> f;
#pragma unroll
    for (int m = 0; m < G::NF; ++m)
        read_frag<BM>(ring, f, 0, m, a_slot[0], b_slot[0], b_toff);

    // the output as a buffer resource: offsets at or past out_bytes are dropped
    const uint32_t out_rows = p.offsets ? p.max_rows : p.rows;
    const uint32_t out_bytes = out_rows * (uint32_t)p.ldc * (MODE == kDown ? 4u : 2u);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(p.C, (short)0, (int)out_bytes, kBufferWord3);

    f32x16 acc[TM][TN];
    int sl = 0;                              // ring slot of the next step (steps done % NS)
    for (int ti = 1;; ++ti) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = f32x16{};
        // The last kAhead steps refill with the next tile's first slices;
        // that tile's A offsets are formed just before (its gathered rows
        // were requested a tile ago and the waits of the steps so far have
        // retired those loads). One call site for the step, so all its
        // requests share one alias scope.
        for (int kt = 0; kt < KT; ++kt) {
            // ring slots: g % NS multiplied, the next one read ahead, the
            // one before (multiplied last step) refilled
            const int sn = sl + 1 == NS ? 0 : sl + 1;
            const int sf = sl == 0 ? NS - 1 : sl - 1;
            uint4 *S = ring + sl * G::STAGE;
            uint4 *Sn = ring + sn * G::STAGE;
            uint4 *Sf = ring + sf * G::STAGE;
            sl = sn;
            ring_step<BM, MODE, NS>(S, Sn, Sf, p, req, kt + kAhead < KT ? kt + kAhead : kt + kAhead - KT,
                                f, acc, a_slot, b_slot, b_toff);
            if (kt == KT - kAhead - 1) {
                // a tile past the end re-requests this one (in bounds, never
                // multiplied)
                if (has_next) {
                    // here and not hoisted to the tile start, where the
                    // gathered rows may not have arrived yet
#pragma unroll
                    for (int i = 0; i < G::AI; ++i)
                        __asm__ volatile("" : "+v"(nraw[i]));
                    a_offsets<BM>(p, nraw, nvalid, req.a_off);
                    b_offsets<BM, MODE>(p, p.b_compact ? s_rank[ne] : ne, nnt, req);
                }
            }
        }

        // ---- epilogue. acc[i][j][r]: token (lane % 32) of token tile i,
        // weight row 8*(r/4) + 4*(lane/32) + r%4 of weight tile j. A lane
        // holds 4-column pieces of one row, so storing from there writes
        // 16 or 32 bytes into each of 32 rows per instruction: partial
        // lines. The results go through a wave-private 4 KB of LDS instead
        // (256-row tiles: an array of its own; 128-row tiles: the stage
        // multiplied last, not refilled before the next tile's first
        // barrier), one 32-row block at a time, and come back as 16-byte
        // pieces of whole rows: every store instruction writes 8 rows of 128
        // bytes (fp32, 32 columns) or 4 to 8 rows of 128 to 256 bytes (bf16).
        // 16-byte chunk c of LDS row r (128-byte rows: half of the 64 banks)
        // sits at chunk c ^ ((r / 2) % 8): the 16 rows a 16-lane write
        // touches, even and odd, then cover every bank once, as do the two
        // rows a 16-lane read touches. Stores past the segment's rows or past N go to an
        // offset the buffer range check drops: no branches. The area is
        // wave-private and 4 KB: a 32-row block of 32 fp32 or 64 bf16
        // columns.
        char *park;
        if constexpr (BM == 256) {
            park = (char *)park_lds + wave * 4096;
        } else {
            // every wave is past its reads of that stage (the requests of
            // the next tile stay in flight)
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            park = (char *)(ring + (sl == 0 ? NS - 1 : sl - 1) * G::STAGE) + wave * 4096;
        }
        const int half = lane >> 5;          // which 4 of each 8 columns the lane holds
        const int prow = lane & 31;          // the row the lane holds
        if (MODE == kDown) {
            const int n0 = nt * kBN + wn * (kBN / 2);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const f32x16 &v = acc[i][j];
                    // 32 rows x 32 fp32: row r at r * 128 bytes, 8 chunks of 4
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int chunk = (2 * gq + half) ^ ((prow >> 1) & 7);
                        park_put16(park, prow * 128 + chunk * 16,
                                   __builtin_bit_cast(u32x4, f32x4{v[4 * gq], v[4 * gq + 1],
                                                                   v[4 * gq + 2], v[4 * gq + 3]}));
                    }
                    const int col = n0 + j * 32 + 4 * (lane & 7);
                    const bool col_ok = col < p.N;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = q * 8 + (lane >> 3);
                        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
                        const u32x4 w4 = park_get16(park, r * 128 + chunk * 16);
                        const int pos = row0 + a_tile_row + i * 32 + r;
                        const uint32_t off = (pos < row_end && col_ok)
                                                 ? ((uint32_t)pos * (uint32_t)p.ldc + col) * 4u
                                                 : out_bytes;
                        __builtin_amdgcn_raw_buffer_store_b128(w4, out_rsrc, off, 0, 0);
                    }
                    fence();
                }
            }
        } else {
            // per 32-row block, two tiles of 32 output columns at a time:
            // bf16, written to LDS as rows of 128 bytes (4 KB per wave),
            // then stored in 16-byte pieces of whole rows
            constexpr int JO = gated(MODE) ? TN / 2 : TN;     // output column tiles
            static_assert(JO % 2 == 0, "output column tiles come in pairs");
            const int ncols = gated(MODE) ? p.I : p.N;
            const int n0 = nt * (gated(MODE) ? kBN / 2 : kBN) +
                           wn * (gated(MODE) ? kBN / 4 : kBN / 2);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int jp = 0; jp < JO; jp += 2) {
                    uint32_t hv[2][8];           // bf16 pairs, the lane's columns of each tile
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = jp + jj;
                        // the tile's accumulators into VGPRs, one read each:
                        // written out, so the compiler does not move every
                        // accumulator of the tile list at once (which spills)
                        f32x16 gv, uv;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(gv[r]) : "a"(acc[i][j][r]));
                            if (gated(MODE))
                                __asm__ volatile("v_accvgpr_read_b32 %0, %1"
                                                 : "=v"(uv[r])
                                                 : "a"(acc[i][j + TN / 2][r]));
                        }
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            constexpr bool LIM = MODE == kGateUpLimit;
                            const float x0 = gated(MODE)
                                                 ? swiglu<LIM>(gv[2 * c], uv[2 * c], p.limit)
                                                 : relu_sq(gv[2 * c]);
                            const float x1 = gated(MODE)
                                                 ? swiglu<LIM>(gv[2 * c + 1], uv[2 * c + 1], p.limit)
                                                 : relu_sq(gv[2 * c + 1]);
                            hv[jj][c] = pack_bf16x2(x0, x1);
                        }
                    }
                    // the pair's rows into LDS: tile jj's columns 8 gq + 4 half
                    // .. + 3 are bytes 16 (4 jj + gq) + 8 half of the row
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const int chunk = (4 * jj + gq) ^ ((prow >> 1) & 7);
                            park_put8(park, prow * 128 + chunk * 16 + 8 * half,
                                      u32x2{hv[jj][2 * gq], hv[jj][2 * gq + 1]});
                        }
                    // and out in 16-byte pieces of whole rows (8 per row)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = q * 8 + (lane >> 3), c = lane & 7;
                        const int chunk = c ^ ((r >> 1) & 7);
                        const u32x4 w4 = park_get16(park, r * 128 + chunk * 16);
                        const int pos = row0 + a_tile_row + i * 32 + r;
                        const int col = n0 + jp * 32 + 8 * c;
                        const uint32_t off = (pos < row_end && col < ncols)
                                                 ? ((uint32_t)pos * (uint32_t)p.ldc + col) * 2u
                                                 : out_bytes;
                        __builtin_amdgcn_raw_buffer_store_b128(w4, out_rsrc, off, 0, 0);
                    }
                    fence();
                }
            }
        }

        if (!has_next)
            break;
        e = ne;
        row0 = nrow0;
        row_end = nrow_end;
        nt = nnt;
        has_next = place<BM>(tl, ti + 1, ne, nrow0, nrow_end, nnt);
        nvalid = gathered_rows<BM>(p, has_next ? nrow0 : row0, has_next ? nrow_end : row_end, nraw);
    }
    // the requests of the last kAhead stages target LDS this workgroup is
    // about to release
    wait_vmcnt<0>();
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Tiles of the worst case (every segment ragged) for BM-row tiles.
template <int BM, int MODE>
long long tiles_bound(const GemmProblem &p, int &n_tiles) {
    int mt_max;
    if (p.offsets == nullptr) {
        mt_max = (p.rows + BM - 1) / BM;
    } else {
        const int nonempty = p.E < p.max_rows ? p.E : p.max_rows;
        mt_max = (p.max_rows + BM - 1) / BM + nonempty;
    }
    const int n_cols = gated(MODE) ? p.I : p.N;
    const int n_tile = gated(MODE) ? kBN / 2 : kBN;
    n_tiles = (n_cols + n_tile - 1) / n_tile;
    return (long long)mt_max * n_tiles;
}

template <int BM, int MODE>
hipError_t launch_bm(const GemmProblem &p, hipStream_t stream) {
    int n_tiles = 0;
    const long long work = tiles_bound<BM, MODE>(p, n_tiles);
    if (work == 0)
        return hipSuccess;
    // one workgroup per CU, a whole number of XCD rounds, no more than the
    // worst-case tile count needs
    int blocks = cu_count() / kXcds * kXcds;
    if (blocks < kXcds)
        blocks = kXcds;
    const long long need = (work + kXcds - 1) / kXcds * kXcds;
    if (need < blocks)
        blocks = (int)need;
    // the deep ring for 128-row tiles where K has the slices to fill it
    if constexpr (BM == 128) {
        if (p.K / kBK >= kStagesDeep) {
            hipLaunchKernelGGL((k_grouped<BM, MODE, kStagesDeep>), dim3(blocks), dim3(kThreads), 0,
                               stream, p, n_tiles);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_grouped<BM, MODE, kStagesSmall>), dim3(blocks), dim3(kThreads), 0, stream,
                       p, n_tiles);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const GemmProblem &p, hipStream_t stream) {
    int segs = 1;
    if (p.offsets != nullptr)
        segs = p.E < p.max_rows ? p.E : p.max_rows;
    const int rows = p.offsets != nullptr ? p.max_rows : p.rows;
    const int avg = segs > 0 ? rows / segs : 0;
    // 256-row tiles for long segments, unless a dense problem then has fewer
    // tiles than CUs (128-row tiles put twice as many CUs to work)
    int n_tiles = 0;
    if (avg >= 192 && (p.offsets != nullptr || tiles_bound<256, MODE>(p, n_tiles) >= cu_count()))
        return launch_bm<256, MODE>(p, stream);
    return launch_bm<128, MODE>(p, stream);
}

}  // namespace

bool grouped_supported(const GemmProblem &p) {
    // every A offset (rows of A times lda, in bytes) stays below kPastA
    // and every weight offset within one expert, stay below kPastA
    const long long a_rows = p.offsets != nullptr ? p.max_rows : p.rows;
    return !p.affine4 && !p.fp8 && p.scatter == nullptr && p.K % kBK == 0 && p.K / kBK >= kStagesSmall &&
           (p.offsets == nullptr || p.E <= kMaxE) && a_rows * p.lda * 2 < (long long)kPastA &&
           (long long)p.N * p.K * 2 < (long long)kPastA;
}

hipError_t launch_grouped(const GemmProblem &p, hipStream_t stream) {
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp>(p, stream);
    case kGateUpLimit: return launch_mode<kGateUpLimit>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2>(p, stream);
    default: return launch_mode<kDown>(p, stream);
    }
}

}  // namespace moe
