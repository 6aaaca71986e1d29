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

// Weight formats of the tiles: bf16 (or bf16 decoded by a pass before),
// block-FP8 codes, and 4-bit E2M1 codes with NVFP4 (E4M3 per 16) or MXFP4
// (E8M0 per 32) scales.
constexpr int kWBf16 = 0;
constexpr int kWF8 = 1;
constexpr int kWNv4 = 2;
constexpr int kWMx4 = 3;

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

// F8: block-FP8 weights, one byte each in the stages (32-byte rows per
// K-slice instead of 64).
template <int BM, int WF = kWBf16>
struct Geo {
    static constexpr bool F8 = WF == kWF8;
    static constexpr bool F4 = WF == kWNv4 || WF == kWMx4;
    static constexpr int TM = BM / 64;            // 32-token MFMA tiles per wave
    static constexpr int TN = kBN / 64;           // 32-weight-row MFMA tiles per wave
    static constexpr int BROW = F8 ? 2 : F4 ? 1 : 4;  // 16-byte slots per weight row of a stage
    static constexpr int AI = BM * 4 / kThreads;  // A requests per thread per stage
    static constexpr int BI = kBN * BROW / kThreads; // B requests per thread per stage
    static constexpr int PER = AI + BI;
    static constexpr int STAGE = BM * 4 + kBN * BROW;  // 16-byte slots per stage
    static constexpr int NQ = TM * TN;            // MFMAs per sub-step
    static constexpr int NF = TM + TN;            // fragment reads per sub-step (bf16)
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

// Row blocks (p.a_blocked, and p.c_blocked for the bf16 output of the up
// projections): rows in groups of 16, and within a group the 32 columns of
// each K-slice of every row together, so group g's slice ks is 1 KB at
// (g * ld / 32 + ks) * 1 KB, row r of the group at 64 r in it. A request's
// 16 consecutive rows are then one or two 1 KB pieces. The byte offset of
// row r, column c (c within the row of ld elements):
__device__ __forceinline__ uint32_t blocked_offset(uint32_t r, uint32_t c, uint32_t ld) {
    return (r >> 4) * ld * 32u + (c >> 5) * 1024u + (r & 15u) * 64u + (c & 31u) * 2u;
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
        const uint32_t o = p.a_blocked ? blocked_offset((uint32_t)arow, c * 8u, (uint32_t)p.lda)
                                       : ((uint32_t)arow * (uint32_t)p.lda + c * 8) * 2u;
        off[i] = (valid >> i) & 1 ? o : kPastA;
    }
}

// Request state of the tile whose slices are being fetched.
template <int BM, int WF>
struct Req {
    static constexpr bool F8 = WF == kWF8;
    static constexpr bool F4 = Geo<BM, WF>::F4;
    const char *b_base;               // uniform: the expert's weight rows
    uint32_t a_off[Geo<BM>::AI];      // per thread, bytes at K-slice 0
    uint32_t b_off[Geo<BM, WF>::BI];
    uint32_t b_kstep;                 // uniform: bytes from one K-slice to the next (bf16, F8)
    float scale[F8 ? 2 : 1];          // F8: lane b holds the scale of K-block b of each
                                      // weight-row block of the wave (gate, up)
};

// F4: where the scales of this lane's weight rows are (one row per weight
// tile j of the wave): the expert's scale bytes (uniform) and, per j, the
// row's first scale byte.
template <int BM>
struct Scales {
    const uint8_t *base;
    uint32_t off[Geo<BM>::TN];
};

// Which weight row of the expert stage row r (0 .. kBN - 1) of n-tile nt
// holds. A SwiGLU tile holds the gate rows nt * kBN / 2 .. + kBN / 2 - 1,
// then the matching up rows, up_rows after them; any other tile the rows
// nt * kBN .. + kBN - 1. Rows past the matrix are clamped to its last row
// (their outputs are never stored).
__device__ __forceinline__ int tile_weight_row(int r, int nt, bool gate_up, int N, int I,
                                               int up_rows) {
    if (gate_up) {
        int n = nt * (kBN / 2) + (r & (kBN / 2 - 1));
        if (n >= I)
            n = I - 1;
        return r < kBN / 2 ? n : up_rows + n;
    }
    const int wr = nt * kBN + r;
    return wr >= N ? N - 1 : wr;
}

// bf16 stages hold 64 bytes (32 weights along K) of each weight row, four
// 16-byte slots: chunk c of row r sits at slot 4 r + (c xor bits 2..3 of r),
// so a fragment read (16 lanes on 16 consecutive rows, one chunk each)
// covers the 64 banks once. F8 stages hold 32 bytes of each row, two slots:
// chunk c of row r at slot 2 r + (c xor bit 3 of r). The row and chunk of
// slot s:
__device__ __forceinline__ void bf16_slot(int s, int &r, int &c) {
    r = s >> 2;
    c = (s & 3) ^ ((r >> 2) & 3);
}
__device__ __forceinline__ void f8_slot(int s, int &r, int &c) {
    r = s >> 1;
    c = (s & 1) ^ ((r >> 3) & 1);
}

// n-tiles of one expert's weight matrix
__device__ __host__ __forceinline__ int weight_tiles(bool gate_up, int N, int I) {
    return gate_up ? (I + kBN / 2 - 1) / (kBN / 2) : (N + kBN - 1) / kBN;
}

// The weight side of a tile's requests: the expert's base and, per B piece
// of this thread, the byte offset of its row and chunk at K-slice 0 (rows
// past N are clamped to a valid row).
//
// With the tile-packed copy (bf16 or FP8 experts, p.Btiles) the 16 KB (8
// KB) of each K-slice of a tile lie in stage order, so piece s of every
// slice is at 16 s bytes from the slice's start and one request reads 1 KB
// in one piece.
//
// F8 stage rows are 32 bytes, two 16-byte chunks: chunk c of row r sits at
// slot 2 r + (c ^ bit 3 of r). A fragment read (16 lanes, 16 consecutive
// rows, one chunk each) then covers the 64 banks once. The F8 request also
// loads the tile's block scales: for each weight-row block of the wave
// (SwiGLU: the gate rows and the up rows; otherwise the wave's 128 rows),
// lane b takes the scale of K-block b.
template <int BM, int MODE, int WF>
__device__ __forceinline__ void b_offsets(const GemmProblem &p, int e, int nt, Req<BM, WF> &q) {
    using G = Geo<BM, WF>;
    constexpr bool F8 = G::F8;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // segments past the experts: the shared expert's slices (bf16 only)
    const bool sh = !F8 && e >= p.E;
    // weights as stored: 2 bytes (bf16), 1 (FP8) or a half (E2M1) each
    constexpr int kHalfBytes = F8 ? 2 : G::F4 ? 1 : 4;
    q.b_base = sh ? (const char *)(p.B2 + (size_t)(e - p.E) * p.b2_vstride)
                  : (const char *)p.B + (size_t)e * p.N * p.K * kHalfBytes / 2;
    const bool tiles = !G::F4 && !sh && p.Btiles != nullptr && !p.b_compact;
    if (tiles)
        q.b_base = (const char *)p.Btiles + ((size_t)e * weight_tiles(gated(MODE), p.N, p.I) + nt) *
                                                (size_t)p.K * (kBN * kHalfBytes / 2);
    q.b_kstep = (tiles ? kBN : 1) * kBK * kHalfBytes / 2;
    const uint32_t ld = sh ? (uint32_t)p.b2_ld : (uint32_t)p.K;
    const int up_rows = sh ? p.b2_up : p.I;
    if constexpr (F8) {
        const int nb = p.K / 128;           // K-blocks (at most 64: one per lane)
        const int wn = wave & 1;
        const int rb_max = p.N / 128 - 1;
        int rb[2];
        if (gated(MODE)) {
            rb[0] = nt;                     // gate rows nt*128 + wn*64 .. + 63
            rb[1] = p.I / 128 + nt;         // the up rows I + the same
        } else {
            rb[0] = min(nt * 2 + wn, rb_max);  // past N: clamped, never stored
            rb[1] = rb[0];
        }
        const float *sc = (const float *)p.Bscale + (size_t)e * (p.N / 128) * nb;
        const int b = lane < nb ? lane : nb - 1;
#pragma unroll
        for (int g = 0; g < 2; ++g)
            q.scale[g] = sc[(size_t)rb[g] * nb + b];
    }
#pragma unroll
    for (int i = 0; i < G::BI; ++i) {
        const int s = (wave * G::BI + i) * kWave + lane;
        // F4 rows are one 16-byte chunk per K-slice (32 codes)
        int r, c;
        if (G::F4) {
            r = s;
            c = 0;
        } else if (F8) {
            f8_slot(s, r, c);
        } else {
            bf16_slot(s, r, c);
        }
        const int wr = tile_weight_row(r, nt, gated(MODE), p.N, p.I, up_rows);
        q.b_off[i] = tiles ? (uint32_t)s * 16u
                     : G::F4 ? (uint32_t)wr * (ld / 2)
                     : F8 ? (uint32_t)wr * ld + c * 16 : ((uint32_t)wr * ld + c * 8) * 2u;
    }
}

// F4: the weight rows of this lane's fragments (row lane % 32 of each of the
// wave's weight tiles j, mapped as the requests map stage rows) and the
// offsets of their scale bytes: NVFP4 one E4M3 byte per 16 inputs, MXFP4 one
// E8M0 byte per 32, rows of K / 16 or K / 32 bytes.
template <int BM, int MODE, int WF>
__device__ __forceinline__ void scale_rows(const GemmProblem &p, int e, int nt, Scales<BM> &sc) {
    constexpr int TN = Geo<BM>::TN;
    const int lane = threadIdx.x & (kWave - 1);
    const int wn = (threadIdx.x / kWave) & 1;
    const uint32_t row_bytes = (uint32_t)p.K / (WF == kWNv4 ? 16 : 32);
    sc.base = (const uint8_t *)p.Bscale + (size_t)e * p.N * row_bytes;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int wr;
        if (gated(MODE)) {
            // gate rows for j < TN / 2, the matching up rows after them
            const int jj = j < TN / 2 ? j : j - TN / 2;
            int n = nt * (kBN / 2) + wn * (kBN / 4) + jj * 32 + (lane & 31);
            if (n >= p.I)
                n = p.I - 1;
            wr = j < TN / 2 ? n : p.I + n;
        } else {
            wr = nt * kBN + wn * (kBN / 2) + j * 32 + (lane & 31);
            if (wr >= p.N)
                wr = p.N - 1;
        }
        sc.off[j] = (uint32_t)wr * row_bytes;
    }
}

// F4: the 16 scale bytes of block blk of each of this lane's rows (NVFP4:
// 8 K-slices, two bytes each; MXFP4: 16 K-slices, one byte each). Bytes past
// the expert's scales read as zeros (a partial last block).
template <int BM, int WF>
__device__ __forceinline__ void load_scales(const GemmProblem &p, const Scales<BM> &sc, int blk,
                                            u32x4 (&dst)[Geo<BM>::TN]) {
    const uint32_t row_bytes = (uint32_t)p.K / (WF == kWNv4 ? 16 : 32);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(sc.base), (short)0, (int)((uint32_t)p.N * row_bytes), kBufferWord3);
#pragma unroll
    for (int j = 0; j < Geo<BM>::TN; ++j)
        dst[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, sc.off[j] + 16u * (uint32_t)blk, 0, 0));
}

// Piece m (A pieces first, then B pieces) of K-slice ks into one stage.
template <int BM, int MODE, int WF>
__device__ __forceinline__ void request(uint4 *__restrict__ stage, const GemmProblem &p,
                                        const Req<BM, WF> &q, int ks, int m) {
    using G = Geo<BM, WF>;
    constexpr bool F8 = G::F8;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (m < G::AI) {
        // pieces of padding rows (offset kPastA) read as zeros
        const uint32_t kstep = p.a_blocked ? 1024u : kBK * 2;
        buffer_to_lds16(p.A, stage + (wave * G::AI + m) * kWave, q.a_off[m] + (uint32_t)ks * kstep);
    } else {
        const int i = m - G::AI;
        uint32_t kstep;
        if constexpr (G::F4)
            kstep = kBK / 2;
        else
            kstep = q.b_kstep;
        buffer_to_lds16(q.b_base, stage + BM * 4 + (wave * G::BI + i) * kWave,
                        q.b_off[i] + (uint32_t)ks * kstep);
    }
}

// Fragment registers: slot 0 and 1 of a double buffer over sub-steps. F8
// also holds the raw bytes of each weight fragment: 16 bytes per lane, both
// sub-steps of a step (bytes 0-7 sub-step 0, 8-15 sub-step 1).
template <int BM, int WF = kWBf16>
struct Frags {
    bf16x8 a[2][Geo<BM>::TM];
    bf16x8 b[2][Geo<BM>::TN];
    u32x4 braw[WF == kWF8 ? Geo<BM>::TN : 1];
    // F4: 16 codes per lane, 8 for each sub-step (bytes 0-3, then 4-7)
    u32x2 b4[Geo<BM, WF>::F4 ? Geo<BM>::TN : 1];
};

// One 16-byte fragment read of a stage, through a __restrict__ pointer of
// its own (as read_frag): the read then carries an alias scope, which lets
// the compiler tell it from the requests still in flight into other stages.
__device__ __forceinline__ u32x4 lds_frag(const uint4 *__restrict__ S, int slot) {
    return __builtin_bit_cast(u32x4, S[slot]);
}

// Half h (8 bytes) of a 16-byte slot, the same way.
__device__ __forceinline__ u32x2 lds_frag8(const uint4 *__restrict__ S, int slot, int h) {
    return reinterpret_cast<const u32x2 *__restrict__>(S + slot)[h];
}

// Slot `slot`'s weight fragment j from the raw FP8 bytes: e4m3 to bf16 is
// exact (every e4m3 value, NaN included, is a bf16 value); the block scale
// is applied to the fp32 sums, not here.
template <int BM>
__device__ __forceinline__ void cvt_b(Frags<BM, kWF8> &f, int slot, int j) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t w = f.braw[j][2 * slot + q];
        o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
        o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    }
    f.b[slot][j] = __builtin_bit_cast(bf16x8, (u32x4){o[0], o[1], o[2], o[3]});
}

// Slot `slot`'s weight fragment j from the raw E2M1 codes (8 per lane, low
// nibble first) times this lane's scale of them, exactly: an E2M1 value
// times an E4M3 or a power-of-two scale has at most six significant bits.
// MXFP4's power-of-two scale (E8M0, NaN included) is the conversion's own
// scale operand, which multiplies by a power of two exactly; NVFP4's E4M3
// scale is not a power of two, so those codes go to fp32 first, are
// multiplied there and rounded to bf16 (exactly).
template <int BM, int WF>
__device__ __forceinline__ void cvt_b4(Frags<BM, WF> &f, int slot, int j, float scale) {
    const uint32_t w = slot == 0 ? f.b4[j].x : f.b4[j].y;
    uint32_t o[4];
    if constexpr (WF == kWMx4) {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    } else {
        const f32x2_hw v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        const f32x2_hw v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        const f32x2_hw v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        const f32x2_hw v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        o[0] = pack_bf16x2(v0.x * scale, v0.y * scale);
        o[1] = pack_bf16x2(v1.x * scale, v1.y * scale);
        o[2] = pack_bf16x2(v2.x * scale, v2.y * scale);
        o[3] = pack_bf16x2(v3.x * scale, v3.y * scale);
    }
    f.b[slot][j] = __builtin_bit_cast(bf16x8, (u32x4){o[0], o[1], o[2], o[3]});
}

// F4: this lane's scale of the current K-slice from the front of its scale
// block, which then moves on by one slice (MXFP4: one byte; NVFP4: two, of
// which lane half h takes byte h, the 16-input group its K range is in).
template <int WF>
__device__ __forceinline__ float next_scale(u32x4 &blk, int h) {
    constexpr int S = WF == kWNv4 ? 16 : 8;
    const uint32_t b = (WF == kWNv4 ? blk.x >> (8 * h) : blk.x) & 0xffu;
    blk.x = __builtin_amdgcn_alignbit(blk.y, blk.x, S);
    blk.y = __builtin_amdgcn_alignbit(blk.z, blk.y, S);
    blk.z = __builtin_amdgcn_alignbit(blk.w, blk.z, S);
    blk.w = blk.w >> S;
    if constexpr (WF == kWMx4)
        return e8m0_to_f32(b);
    // E4M3 -> bf16 exactly (scale 1), then fp32
    const uint32_t pr = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false));
    return bf16_to_f32(pr & 0xffffu);
}

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
                                          const Req<BM, kWBf16> &q, int ks, Frags<BM> &f,
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
                request<BM, MODE, kWBf16>(Sfill, p, q, ks, m - G::NF);
        }
        fence();
    }
}

// The same step on FP8 weights. The weight fragments of both sub-steps come
// in one 16-byte read per lane (in the previous step's sub-step 1) and are
// converted to bf16 during the step. With that layout, lane half
// h of sub-step kk covers K = 16 h + 8 kk .. + 7 of the slice, so the token
// fragments are read from chunk 2 h + kk.
//
// On the first step of a K-block (`rescale`), each accumulator tile is
// multiplied, just before its first MFMA of the block, by r = (scale of the
// previous K-block) / (scale of this one), per weight-row block of the wave
// (r_gate, r_up): the sums are then kept in units of the current block's
// scale, and the finished sum is multiplied by the last block's scale. That
// is sum_b s_b P_b (P_b the block's exact-weight fp32 partial), with one
// extra rounding per block instead of a second set of accumulators.
template <int BM, int MODE, int NS>
__device__ __forceinline__ void ring_step_f8(const uint4 *__restrict__ S, const uint4 *__restrict__ Snext,
                                             uint4 *__restrict__ Sfill, const GemmProblem &p,
                                             const Req<BM, kWF8> &q, int ks, Frags<BM, kWF8> &f,
                                             f32x16 (&acc)[Geo<BM>::TM][Geo<BM>::TN],
                                             const int (&a_slot)[2], int b_slot, const int *b_toff,
                                             bool rescale, float r_gate, float r_up) {
    using G = Geo<BM, kWF8>;
    constexpr int TM = G::TM, TN = G::TN;
    fence();
    // sub-step 0: MFMAs on slot 0, each weight fragment converted just
    // before its first MFMA; token fragments of sub-step 1 into slot 1 and
    // its weight fragments converted. (Converting slot 0 at the end of the
    // previous step instead makes the compiler wait for every request in
    // flight before the first LDS read of the step.)
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / TN, j = n % TN;
        if (n < TN)
            cvt_b<BM>(f, 0, j);
        if (rescale) {
            const float r = (gated(MODE) && j >= TN / 2) ? r_up : r_gate;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] *= r;
        }
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[0][j], f.a[0][i], acc[i][j], 0, 0, 0);
        if (n < TM)
            f.a[1][n] = __builtin_bit_cast(bf16x8, lds_frag(S, a_slot[1] + n * 128));
        else if (n - TM < TN)
            cvt_b<BM>(f, 1, n - TM);
        fence();
    }
    wait_vmcnt<(NS - 3) * G::PER>();
    __builtin_amdgcn_s_barrier();
    fence();
    // sub-step 1: MFMAs on slot 1; the next step's token fragments and raw
    // weight bytes, and the refill of the stage read in the previous step
    constexpr int NM = TM + TN + G::PER;
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / TN, j = n % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[1][j], f.a[1][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int m = n * NM / G::NQ; m < (n + 1) * NM / G::NQ; ++m) {
            if (m < TM)
                f.a[0][m] = __builtin_bit_cast(bf16x8, lds_frag(Snext, a_slot[0] + m * 128));
            else if (m < TM + TN)
                f.braw[m - TM] = lds_frag(Snext, b_slot + b_toff[m - TM]);
            else
                request<BM, MODE, kWF8>(Sfill, p, q, ks, m - TM - TN);
        }
        fence();
    }
}

// The same step on 4-bit E2M1 weights. The codes of both sub-steps come in
// one 8-byte read per lane and weight tile (in the previous step's sub-step
// 1); lane half h of sub-step kk covers K = 16 h + 8 kk .. + 7 of the slice,
// as for FP8, and sc[j] is this lane's scale of its row of tile j in the
// slice. `late`: scale loads were issued after the requests of the stage
// waited for here, so TN more loads may still be in flight.
template <int BM, int MODE, int NS, int WF>
__device__ __forceinline__ void ring_step_f4(const uint4 *__restrict__ S, const uint4 *__restrict__ Snext,
                                             uint4 *__restrict__ Sfill, const GemmProblem &p,
                                             const Req<BM, WF> &q, int ks, Frags<BM, WF> &f,
                                             f32x16 (&acc)[Geo<BM>::TM][Geo<BM>::TN],
                                             const int (&a_slot)[2], int b_slot, const int *b_toff,
                                             const float (&sc)[Geo<BM>::TN], bool late) {
    using G = Geo<BM, WF>;
    constexpr int TM = G::TM, TN = G::TN;
    const int h = (threadIdx.x & (kWave - 1)) >> 5;
    fence();
    // sub-step 0: MFMAs on slot 0, each weight fragment converted just
    // before its first MFMA; token fragments of sub-step 1 into slot 1 and
    // its weight fragments converted
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / TN, j = n % TN;
        if (n < TN)
            cvt_b4<BM, WF>(f, 0, j, sc[j]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[0][j], f.a[0][i], acc[i][j], 0, 0, 0);
        if (n < TM) {
            f.a[1][n] = __builtin_bit_cast(bf16x8, lds_frag(S, a_slot[1] + n * 128));
        } else if (n - TM < TN) {
            cvt_b4<BM, WF>(f, 1, n - TM, sc[n - TM]);
            // here, between these MFMAs: left alone, the compiler sinks the
            // conversions to their first use, all of them after the last
            // MFMA of the sub-step, where the next MFMAs wait for them
            __asm__ volatile("" : "+v"(f.b[1][n - TM]));
        }
        fence();
    }
    if (late)
        wait_vmcnt<(NS - 3) * G::PER + TN>();
    else
        wait_vmcnt<(NS - 3) * G::PER>();
    __builtin_amdgcn_s_barrier();
    fence();
    // sub-step 1: MFMAs on slot 1; the next step's token fragments and
    // codes, and the refill of the stage read in the previous step
    constexpr int NM = TM + TN + G::PER;
#pragma unroll
    for (int n = 0; n < G::NQ; ++n) {
        const int i = n / TN, j = n % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[1][j], f.a[1][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int m = n * NM / G::NQ; m < (n + 1) * NM / G::NQ; ++m) {
            if (m < TM)
                f.a[0][m] = __builtin_bit_cast(bf16x8, lds_frag(Snext, a_slot[0] + m * 128));
            else if (m < TM + TN)
                f.b4[m - TM] = lds_frag8(Snext, b_slot + b_toff[m - TM], h);
            else
                request<BM, MODE, WF>(Sfill, p, q, ks, m - TM - TN);
        }
        fence();
    }
}

// Prologue: the first NS - 1 slices of the first tile into stages 0 ..
// NS - 2.
template <int BM, int MODE, int NS, int WF>
__device__ __forceinline__ void prime(uint4 *__restrict__ ring, const GemmProblem &p,
                                      const Req<BM, WF> &q) {
    using G = Geo<BM, WF>;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
#pragma unroll
        for (int m = 0; m < G::PER; ++m)
            request<BM, MODE, WF>(ring + st * G::STAGE, p, q, st, m);
}

template <int BM, int MODE, int NS, int WF>
__global__ __launch_bounds__(kThreads, 1) void k_grouped(GemmProblem p, int n_tiles) {
    using G = Geo<BM, WF>;
    constexpr bool F8 = G::F8;
    constexpr bool F4 = G::F4;
    // F4: K-slices per scale block (16 bytes of a row's scales)
    constexpr int SBS = WF == kWNv4 ? 8 : 16;
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
    const int nseg = p.offsets ? p.E + p.E2 : 1;
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
    Req<BM, WF> req;                         // the tile being fetched
    {
        int raw[G::AI];
        const int valid = gathered_rows<BM>(p, row0, row_end, raw);
        a_offsets<BM>(p, raw, valid, req.a_off);
        b_offsets<BM, MODE, WF>(p, p.b_compact && e < p.E ? s_rank[e] : e, nt, req);
    }
    int ne, nrow0, nrow_end, nnt;            // the next tile (if any)
    bool has_next = place<BM>(tl, 1, ne, nrow0, nrow_end, nnt);
    // F4: the scale rows of this tile and the next, and this lane's scale
    // blocks: the one being used (shifted on by a K-slice each step) and the
    // one after it, loaded a block ahead (the first one here, before the
    // first requests, so the first wait for it is a short one)
    Scales<BM> scs, nscs;
    u32x4 scur[F4 ? TN : 1], snext[F4 ? TN : 1];
    if constexpr (F4) {
        scale_rows<BM, MODE, WF>(p, e, nt, scs);
        load_scales<BM, WF>(p, scs, 0, scur);
    }
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
        // F8, F4: lane half h of sub-step kk covers chunk 2 h + kk of the slice
        const int ch = F8 || F4 ? 2 * (lane >> 5) + kk : kk * 2 + (lane >> 5);
        a_slot[kk] = slot_of(a_tile_row + (lane & 31), ch);
        b_slot[kk] = BM * 4 + slot_of(b_row0 + (lane & 31), ch);
    }
    if constexpr (F8) {
        // the lane's 16-byte chunk (lane / 32) of its 32-byte row; tiles 32
        // rows apart keep the swizzle
        const int rr = b_row0 + (lane & 31);
        b_slot[0] = BM * 4 + rr * 2 + ((lane >> 5) ^ ((rr >> 3) & 1));
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b_toff[j] /= 2;
    }
    if constexpr (F4) {
        // the lane's row, one 16-byte slot of 32 codes (lane half h reads
        // its 8 bytes 8 h ..)
        b_slot[0] = BM * 4 + b_row0 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b_toff[j] /= 4;
    }

    const int KT = p.K / kBK;
    prime<BM, MODE, NS, WF>(ring, p, req);
    wait_vmcnt<(NS - 2) * G::PER>();
    __builtin_amdgcn_s_barrier();
    Frags<BM, WF> f;
    if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.a[0][i] = __builtin_bit_cast(bf16x8, ring[a_slot[0] + i * 128]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            f.braw[j] = __builtin_bit_cast(u32x4, ring[b_slot[0] + b_toff[j]]);
    } else if constexpr (F4) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.a[0][i] = __builtin_bit_cast(bf16x8, ring[a_slot[0] + i * 128]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            f.b4[j] = lds_frag8(ring, b_slot[0] + b_toff[j], lane >> 5);
    } else {
#pragma unroll
        for (int m = 0; m < G::NF; ++m)
            read_frag<BM>(ring, f, 0, m, a_slot[0], b_slot[0], b_toff);
    }

    // Each tile stores through a buffer resource based at its own first
    // output row and spanning its rows that lie in the segment: offsets stay
    // below BM rows of ldc elements (< 2^26 bytes) however large the output
    // is, and an offset at or past the span (padding rows, columns past N)
    // is dropped by the range check.
    constexpr uint32_t kElt = MODE == kDown ? 4u : 2u;
    const uint32_t kDropped = 0x80000000u;   // past every tile's span

    f32x16 acc[TM][TN];
    int sl = 0;                              // ring slot of the next step (steps done % NS)
    int late = 0;                            // F4: steps whose wait allows the scale loads
    for (int ti = 1;; ++ti) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = f32x16{};
        // F8: this tile's block scales (lane b: K-block b) and the units the
        // sums are kept in (the scale of the K-block being multiplied)
        float sc_gate = 0.0f, sc_up = 0.0f, rho_gate = 0.0f, rho_up = 0.0f;
        if constexpr (F4) {
            if (has_next)
                scale_rows<BM, MODE, WF>(p, ne, nnt, nscs);
            else
                nscs = scs;                  // loaded again, never used
        }
        if constexpr (F8) {
            sc_gate = req.scale[0];
            sc_up = req.scale[1];
            rho_gate = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_gate), 0));
            rho_up = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_up), 0));
        }
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
            const int ks = kt + kAhead < KT ? kt + kAhead : kt + kAhead - KT;
            if constexpr (F8) {
                // first step of K-block b > 0: r = (previous block's scale) /
                // (this block's scale); uniform. The step index passes through
                // an empty asm so the loop is not peeled at kt = 0: a second
                // inlined copy of the step makes the compiler wait for every
                // request in flight before its LDS reads.
                int kq = kt;
                __asm__ volatile("" : "+s"(kq));
                const bool rescale = kq > 0 && (kq & 3) == 0;
                float r_gate = 1.0f, r_up = 1.0f;
                if (rescale) {
                    const int b = kq >> 2;
                    const float s_gate = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_gate), b));
                    r_gate = rho_gate / s_gate;
                    rho_gate = s_gate;
                    if (gated(MODE)) {
                        const float s_up = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_up), b));
                        r_up = rho_up / s_up;
                        rho_up = s_up;
                    }
                }
                ring_step_f8<BM, MODE, NS>(S, Sn, Sf, p, req, ks, f, acc, a_slot, b_slot[0], b_toff,
                                           rescale, r_gate, r_up);
            } else if constexpr (F4) {
                // at the start of each scale block the next block's loads
                // (this tile's, or the next tile's first): issued after the
                // requests of the next two stages waited for, so those two
                // waits allow TN more loads in flight
                if (kt % SBS == 0) {
                    const int nb = kt / SBS + 1;
                    if (nb * SBS < KT)
                        load_scales<BM, WF>(p, scs, nb, snext);
                    else
                        load_scales<BM, WF>(p, nscs, 0, snext);
                    late = 2;
                }
                float sc[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    sc[j] = next_scale<WF>(scur[j], lane >> 5);
                ring_step_f4<BM, MODE, NS, WF>(S, Sn, Sf, p, req, ks, f, acc, a_slot, b_slot[0], b_toff,
                                               sc, late > 0);
                late = late > 0 ? late - 1 : 0;
                if (kt % SBS == SBS - 1 || kt == KT - 1) {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        scur[j] = snext[j];
                }
            } else {
                ring_step<BM, MODE, NS>(S, Sn, Sf, p, req, ks, f, acc, a_slot, b_slot, b_toff);
            }
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
                    b_offsets<BM, MODE, WF>(p, p.b_compact && ne < p.E ? s_rank[ne] : ne, nnt, req);
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
        // a per-expert scale of the sums (NVFP4's global scale), uniform
        const bool gscaled = !F8 && p.Bglobal != nullptr && e < p.E;
        const float gsc = gscaled ? p.Bglobal[e] : 1.0f;
        const int span_rows = min(row_end - row0, BM);
        // row blocks: based at the block of row0, spanning the blocks of the
        // tile's rows (rows past row_end are dropped by their offset)
        const bool cb = MODE != kDown && p.c_blocked;
        const int row_base = cb ? row0 & ~15 : row0;
        const uint32_t span_bytes =
            cb ? (uint32_t)(((row0 + span_rows + 15) & ~15) - row_base) * (uint32_t)p.ldc * 2u
               : (uint32_t)span_rows * (uint32_t)p.ldc * kElt;
        const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (char *)p.C + (size_t)row_base * (size_t)p.ldc * kElt, (short)0, (int)span_bytes,
            kBufferWord3);
        if (MODE == kDown) {
            const int n0 = nt * kBN + wn * (kBN / 2);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    // the tile's accumulators into VGPRs one read each (F8:
                    // the finished sum in units of the last block's scale);
                    // a whole-vector copy lets the compiler move every
                    // accumulator of the tile list at once, which spills
                    f32x16 v;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if constexpr (F8)
                            v[r] = acc[i][j][r] * rho_gate;
                        else
                            __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[r]) : "a"(acc[i][j][r]));
                    }
                    if (gscaled)
                        v = v * gsc;
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
                        const int prel = a_tile_row + i * 32 + r;   // row within the tile
                        const uint32_t off = (row0 + prel < row_end && col_ok)
                                                 ? ((uint32_t)prel * (uint32_t)p.ldc + col) * 4u
                                                 : kDropped;
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
                            if constexpr (F8) {
                                gv[r] = acc[i][j][r] * rho_gate;
                                if (gated(MODE))
                                    uv[r] = acc[i][j + TN / 2][r] * rho_up;
                            } else {
                                __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(gv[r]) : "a"(acc[i][j][r]));
                                if (gated(MODE))
                                    __asm__ volatile("v_accvgpr_read_b32 %0, %1"
                                                     : "=v"(uv[r])
                                                     : "a"(acc[i][j + TN / 2][r]));
                            }
                        }
                        if (gscaled) {
                            gv = gv * gsc;
                            if (gated(MODE))
                                uv = uv * gsc;
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
                        const int prel = a_tile_row + i * 32 + r;   // row within the tile
                        const int col = n0 + jp * 32 + 8 * c;
                        const uint32_t at =
                            cb ? blocked_offset((uint32_t)(row0 - row_base + prel), (uint32_t)col,
                                                (uint32_t)p.ldc)
                               : ((uint32_t)prel * (uint32_t)p.ldc + col) * 2u;
                        const uint32_t off = (row0 + prel < row_end && col < ncols) ? at : kDropped;
                        __builtin_amdgcn_raw_buffer_store_b128(w4, out_rsrc, off, 0, 0);
                    }
                    fence();
                }
            }
        }

        if (!has_next)
            break;
        if constexpr (F4)
            scs = nscs;
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
        const int segs = p.E + p.E2;
        const int nonempty = segs < p.max_rows ? segs : p.max_rows;
        mt_max = (p.max_rows + BM - 1) / BM + nonempty;
    }
    const int n_cols = gated(MODE) ? p.I : p.N;
    const int n_tile = gated(MODE) ? kBN / 2 : kBN;
    n_tiles = (n_cols + n_tile - 1) / n_tile;
    return (long long)mt_max * n_tiles;
}

template <int BM, int MODE, int WF = kWBf16>
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
            hipLaunchKernelGGL((k_grouped<BM, MODE, kStagesDeep, WF>), dim3(blocks), dim3(kThreads), 0,
                               stream, p, n_tiles);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_grouped<BM, MODE, kStagesSmall, WF>), dim3(blocks), dim3(kThreads), 0, stream,
                       p, n_tiles);
    return hipGetLastError();
}

#if !defined(MOE_GROUPED_F8_UNIT) && !defined(MOE_GROUPED_F4_UNIT)
// The tile-packed copy of a weight tensor W [E][N][K] of bf16 (esz 2) or
// FP8 codes (esz 1): tiles[e][nt][ks] is what K-slice ks of n-tile nt puts
// into a stage (16 or 8 KB), slot s (16 bytes) at 16 s. One thread per
// slot, read from W as the requests of the standard layout read it.
__global__ __launch_bounds__(kThreads) void k_pack_tiles(const char *__restrict__ W,
                                                         uint4 *__restrict__ tiles, int E, int N,
                                                         int K, int I, int gate_up, int esz) {
    const int nts = weight_tiles(gate_up != 0, N, I);
    const int KS = K / kBK;
    const int slots = kBN * 2 * esz;
    const size_t total = (size_t)E * nts * KS * slots;
    for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * kThreads) {
        const int s = (int)(idx % slots);
        size_t rest = idx / slots;
        const int ks = (int)(rest % KS);
        rest /= KS;
        const int nt = (int)(rest % nts);
        const int e = (int)(rest / nts);
        int r, c;
        if (esz == 2)
            bf16_slot(s, r, c);
        else
            f8_slot(s, r, c);
        const int wr = tile_weight_row(r, nt, gate_up != 0, N, I, I);
        const size_t src = (((size_t)e * N + wr) * K + (size_t)ks * kBK) * esz + (size_t)c * 16;
        tiles[idx] = *(const uint4 *)(W + src);
    }
}

template <int MODE>
hipError_t launch_mode(const GemmProblem &p, hipStream_t stream) {
    int segs = 1;
    if (p.offsets != nullptr)
        segs = p.E + p.E2 < p.max_rows ? p.E + p.E2 : p.max_rows;
    const int rows = p.offsets != nullptr ? p.max_rows : p.rows;
    const int avg = segs > 0 ? rows / segs : 0;
    // 256-row tiles for long segments, unless a dense problem then has fewer
    // tiles than CUs (128-row tiles put twice as many CUs to work)
    int n_tiles = 0;
    if (avg >= 192 && (p.offsets != nullptr || tiles_bound<256, MODE>(p, n_tiles) >= cu_count()))
        return launch_bm<256, MODE>(p, stream);
    // The down projection of a routed batch takes them from 64 rows per
    // segment on when they still fill two rounds of CUs: at 96 rows over 130
    // segments (the relu^2 block, T = 2048, E = 128, k = 6, its shared expert
    // as two segments) 256-row tiles ran 363 us against 401 us for 128-row
    // tiles, where the up projection went the other way (408 against 392 us);
    // at 128 rows over 32 segments, four of them long (the 4-bit block at
    // T = 1024), they left CUs idle: 55 against 50 us
    if (MODE == kDown && p.offsets != nullptr && avg >= 64 &&
        tiles_bound<256, MODE>(p, n_tiles) >= 2LL * cu_count())
        return launch_bm<256, MODE>(p, stream);
    return launch_bm<128, MODE>(p, stream);
}

#endif

}  // namespace

#if defined(MOE_GROUPED_F4_UNIT)
// NVFP4 and MXFP4 weights: 256-row tiles (the scales are applied as the
// codes are converted, so the accumulators need no rescaling and stay in
// AGPRs, as for bf16)
hipError_t launch_grouped_f4(const GemmProblem &p, hipStream_t stream) {
    if (p.nvfp4) {
        switch (p.mode) {
        case kGateUp: return launch_bm<256, kGateUp, kWNv4>(p, stream);
        case kGateUpLimit: return launch_bm<256, kGateUpLimit, kWNv4>(p, stream);
        case kUpRelu2: return launch_bm<256, kUpRelu2, kWNv4>(p, stream);
        default: return launch_bm<256, kDown, kWNv4>(p, stream);
        }
    }
    switch (p.mode) {
    case kGateUp: return launch_bm<256, kGateUp, kWMx4>(p, stream);
    case kGateUpLimit: return launch_bm<256, kGateUpLimit, kWMx4>(p, stream);
    case kUpRelu2: return launch_bm<256, kUpRelu2, kWMx4>(p, stream);
    default: return launch_bm<256, kDown, kWMx4>(p, stream);
    }
}
#elif defined(MOE_GROUPED_F8_UNIT)
// FP8 weights: 128-row tiles, whose 128 accumulators per lane stay in VGPRs
// (this unit is compiled with the MFMAs' VGPR form) so the per-K-block
// rescale is one multiply per accumulator; the raw weight bytes fit beside
// them.
hipError_t launch_grouped_f8(const GemmProblem &p, hipStream_t stream) {
    switch (p.mode) {
    case kGateUp: return launch_bm<128, kGateUp, kWF8>(p, stream);
    case kGateUpLimit: return launch_bm<128, kGateUpLimit, kWF8>(p, stream);
    case kUpRelu2: return launch_bm<128, kUpRelu2, kWF8>(p, stream);
    default: return launch_bm<128, kDown, kWF8>(p, stream);
    }
}
#else
bool grouped_supported(const GemmProblem &p) {
    // every A offset (rows of A times lda, in bytes) and every weight offset
    // within one expert stay below kPastA; the rows of a gathered A are the
    // positions divided by gather_div (the tokens of the up projection)
    long long a_rows = p.offsets != nullptr ? p.max_rows : p.rows;
    if (p.gather != nullptr && p.gather_div > 1)
        a_rows = (a_rows + p.gather_div - 1) / p.gather_div;
    // FP8: 128 x 128 scale blocks (a gated N splits at I, a multiple of 128),
    // at most 64 K-blocks (one per lane), the caller's weights as stored
    const bool fp8_ok = !p.fp8 || (p.K % 128 == 0 && p.K / 128 <= kWave && p.N % 128 == 0 &&
                                   (!gated(p.mode) || p.I % 128 == 0) && !p.b_compact);
    // shared segments: bf16 weights beside bf16 (or decoded) experts, every
    // weight offset of a slice below kPastA
    const long long b2_rows = gated(p.mode) ? (long long)p.b2_up + p.I : p.N;
    // NVFP4, MXFP4: the caller's codes and scales as stored, no shared
    // segments (the shared expert's weights are bf16)
    const bool f4 = p.nvfp4 || p.mxfp4;
    const bool f4_ok = !f4 || (p.E2 == 0 && !p.b_compact && p.Bscale != nullptr);
    const bool e2_ok = p.E2 == 0 ||
                       (p.E2 > 0 && !p.fp8 && !f4 && p.offsets != nullptr && p.B2 != nullptr &&
                        b2_rows * p.b2_ld * 2 < (long long)kPastA && p.b2_ld >= p.K);
    const long long b_bytes = p.fp8 ? (long long)p.N * p.K : f4 ? (long long)p.N * p.K / 2
                                                                : (long long)p.N * p.K * 2;
    return !p.affine4 && fp8_ok && f4_ok && e2_ok && p.scatter == nullptr && p.K % kBK == 0 &&
           p.K / kBK >= kStagesSmall && (p.offsets == nullptr || p.E + p.E2 <= kMaxE) &&
           a_rows * p.lda * 2 < (long long)kPastA && b_bytes < (long long)kPastA;
}

size_t pack_tiles_bytes(int E, int N, int K, int I, bool gate_up, int esz) {
    return (size_t)E * weight_tiles(gate_up, N, I) * (size_t)K * kBN * esz;
}

hipError_t launch_pack_tiles(const void *w, void *tiles, int E, int N, int K, int I, bool gate_up,
                             int esz, hipStream_t stream) {
    if (E == 0)
        return hipSuccess;
    if (K % kBK != 0 || (gate_up && N != 2 * I) || (esz != 1 && esz != 2))
        return hipErrorInvalidValue;
    const size_t slots = pack_tiles_bytes(E, N, K, I, gate_up, esz) / 16;
    const size_t want = (slots + kThreads - 1) / kThreads;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(k_pack_tiles, dim3(blocks), dim3(kThreads), 0, stream, (const char *)w,
                       (uint4 *)tiles, E, N, K, I, gate_up ? 1 : 0, esz);
    return hipGetLastError();
}

hipError_t launch_grouped(const GemmProblem &p, hipStream_t stream) {
    if (p.fp8)
        return launch_grouped_f8(p, stream);
    if (p.nvfp4 || p.mxfp4)
        return launch_grouped_f4(p, stream);
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp>(p, stream);
    case kGateUpLimit: return launch_mode<kGateUpLimit>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2>(p, stream);
    default: return launch_mode<kDown>(p, stream);
    }
}
#endif

}  // namespace moe
