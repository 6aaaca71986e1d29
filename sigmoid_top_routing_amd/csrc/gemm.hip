// gemm.hip -- grouped expert GEMMs on bf16 MFMA (gfx950).
//
// One launch multiplies every expert segment by its expert's weight:
//   C[p, n] = sum_k A[row(p), k] * B[e(p), n, k]   (fp32 accumulate)
// where the positions p of expert e are offsets[e] .. offsets[e+1]-1 of the
// plan. Both operands are K-contiguous ("NT"), the layout of the pages'
// weights: gate_up (E, 2I, H) with gate rows first and down (E, H, I)
// (TileGym PR #187, "Weight layout and routing").
//
// Epilogues, all in fp32 on the accumulators and rounded once on the store
// (vllm.cpp PR #684, W2 commit: widen, compute, round once):
//   kGateUp  h[p, n] = bf16(silu(g) * u), g = C[p, n], u = C[p, I + n]
//   kUpRelu2 h[p, n] = bf16((u < 0 ? 0 : u)^2), u = C[p, n]
//                      (bloomery PR #235: relu^2 keeps non-finite inputs)
//   kDown    y[scatter[p], n] = C[p, n] in fp32, back in assignment order
//
// Which kernel. bf16 weights with K a multiple of 32 and at least 128 go to
// the persistent direct-to-LDS kernel of grouped_gemm.hip. This file holds
// the register-staged kernel for the rest: the 4-bit affine weights, whose
// codes are decoded (scale * q + bias, group 64) to bf16 between the global
// load and the LDS store, and short or odd K.
//
// Tiling. A workgroup of 4 waves owns a BM x 256 tile of one expert and
// walks K in steps of 64. Per step it stages the A rows (gathered through
// the plan: row(p) = gather[p] / gather_div, so x is never permuted in
// memory) and the 256 weight rows in LDS, double buffered, with a 16-byte
// XOR swizzle so the MFMA operand reads hit distinct banks. Each wave owns
// a (BM/2) x 128 quarter and issues v_mfma_f32_32x32x16_bf16 over it.
// For kGateUp a tile's weight rows are 128 gate rows and the 128 up rows
// that pair with them, and each wave takes matching gate and up columns, so
// silu(g) * u is formed in registers without an LDS exchange.
//
// Tile order. Workgroups are dispatched to the 8 XCDs round robin, so the
// block index is remapped to give each XCD an equal contiguous run of the
// real tiles in m-major, n-minor order: the workgroups resident on an XCD at
// one time are the n-tiles of one or two m-tiles, which read the same A rows
// and (an expert's m-tiles being adjacent) the same weight rows from its L2.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kXcds = 8;

// 8 chunks of 16 bytes per row of 64 bf16. A ds_read_b128 serves 16 lanes
// per pass from 64 banks (256 bytes); the fragment reads of 16 consecutive
// rows then fall in distinct 16-byte bank groups when the chunk is XORed
// with bits 1-3 of the row (bit 0 already picks the 128-byte half).
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 8 + (chunk ^ ((row >> 1) & 7));
}

// Which tile this workgroup owns: the expert, the BM rows of its segment
// and the n-tile. The real tiles (sum over experts of ceil(rows_e / BM),
// times n_tiles) are numbered m-major, n-minor, and each XCD takes an equal
// contiguous share of that numbering: workgroups reach the XCDs round robin
// (XCD = block % 8) and each XCD starts its workgroups in block order, so the
// workgroups resident on one XCD at a time are the n-tiles of one or two
// m-tiles, which share the A rows and the expert's weight rows in that XCD's
// L2. The grid is sized for the worst case; workgroups past the real tiles
// return at once. Returns false for those.
template <int BM>
__device__ bool locate_tile(const GemmProblem &p, int n_tiles, int *e_out, int *row0,
                            int *row_end, int *nt_out) {
    __shared__ int s_wsum[4];
    __shared__ int s_hit[3];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    int tiles = 0, lo = 0, hi = 0;
    if (p.offsets == nullptr) {
        if (tid == 0) {
            hi = p.rows;
            tiles = (p.rows + BM - 1) / BM;
        }
    } else if (tid < p.E) {
        lo = p.offsets[tid];
        hi = p.offsets[tid + 1];
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
    if (tid == 0)
        s_hit[0] = -1;
    __syncthreads();
    int total = 0;
    for (int w = 0; w < 4; ++w) {
        if (w < wave)
            incl += s_wsum[w];
        total += s_wsum[w];
    }
    const int excl = incl - tiles;
    const int work = total * n_tiles;
    const int share = (work + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int L = (blockIdx.x % kXcds) * share + slot;
    if (slot >= share || L >= work)
        return false;                       // uniform over the workgroup
    const int mt = L / n_tiles;
    if (tiles > 0 && mt >= excl && mt < incl) {
        s_hit[0] = tid;
        s_hit[1] = lo + (mt - excl) * BM;
        s_hit[2] = hi;
    }
    __syncthreads();
    *e_out = s_hit[0];
    *row0 = s_hit[1];
    *row_end = s_hit[2];
    *nt_out = L % n_tiles;
    return true;
}

// worst-case number of m-tiles, then the grid: a whole number of XCD rounds
// that covers every real tile
template <int BM>
int grid_blocks(const GemmProblem &p, int n_tiles) {
    int mt_max;
    if (p.offsets == nullptr) {
        mt_max = (p.rows + BM - 1) / BM;
    } else {
        const int nonempty = p.E < p.max_rows ? p.E : p.max_rows;
        mt_max = (p.max_rows + BM - 1) / BM + nonempty;
    }
    const int work = mt_max * n_tiles;
    return (work + kXcds - 1) / kXcds * kXcds;
}

// Main loop. A step covers K = 64 in 4 sub-steps of K = 16; a sub-step is
// TM * TN independent MFMAs, and every memory instruction of the step is
// placed between two of them so that it issues while the matrix core is
// busy (scheduling fences keep the written order):
//   sub-step 0, 1, 2: LDS reads of the next sub-step's fragments (into the
//                     other half of a register double buffer)
//   sub-step 2:       also the LDS writes of the staged registers (operands
//                     of step kt + 1) into the idle LDS buffer
//   barrier           (the idle buffer is now complete; the current one is
//                     no longer read)
//   sub-step 3:       LDS reads of step kt + 1's first fragments, and the
//                     global loads of step kt + 2 into the staged registers
// So the global loads have sub-steps 3, 0 and 1 to arrive and the LDS reads
// a whole sub-step. The loop body has no branches: rows past a segment or
// past N are clamped to a valid row (their results are never stored) and
// loads past the last step reload it.
//
// Global addresses are a uniform base (the operand, or the expert's weight
// matrix) plus a 32-bit byte offset per thread; the host limits keep every
// operand and every expert's matrix under 2^32 bytes.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint4 load16(const char *base, uint32_t off) {
    return *reinterpret_cast<const uint4 *>(base + off);
}

template <int BM, int MODE, bool AFF>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmProblem p, int n_tiles) {
    constexpr int BN = 256;
    constexpr int TM = BM / 64;          // 32-row MFMA tiles per wave
    constexpr int TN = BN / 64;          // 32-col MFMA tiles per wave
    constexpr int AR = BM / 32;          // A rows staged per thread per step
    constexpr int BR = BN / 32;          // B rows staged per thread per step (bf16)
    constexpr int BQ = BN / 128;         // B half-rows per thread per step (affine-4)
    constexpr int BLOADS = AFF ? BQ : BR;
    constexpr int STAGE = (BM + BN) * 8; // 16-byte slots per LDS buffer
    static_assert(TN % 2 == 0, "gate and up columns come in pairs");

    __shared__ uint4 smem[2 * STAGE];
    __shared__ int s_out_row[BM];

    int e, row0, row_end, nt;
    if (!locate_tile<BM>(p, n_tiles, &e, &row0, &row_end, &nt))
        return;
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row_end = __builtin_amdgcn_readfirstlane(row_end);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int n_out0 = nt * (gated(MODE) ? BN / 2 : BN);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int chunk = tid & 7;

    if (MODE == kDown) {
        for (int r = tid; r < BM; r += kThreads) {
            const int pos = row0 + r;
            s_out_row[r] = pos < row_end ? (p.scatter ? p.scatter[pos] : pos) : -1;
        }
    }

    // ---- A rows this thread stages (clamped into the segment)
    const char *a_base = (const char *)p.A;
    uint32_t a_off[AR];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
        int pos = row0 + (tid >> 3) + i * 32;
        if (pos >= row_end)
            pos = row_end - 1;
        const int arow = p.gather ? p.gather[pos] / p.gather_div : pos;
        a_off[i] = ((uint32_t)arow * (uint32_t)p.lda + chunk * 8) * 2u;
    }

    // ---- B rows this thread stages (clamped below N), relative to expert e
    auto b_row = [&](int r) -> int {
        if (gated(MODE)) {
            int n = n_out0 + (r % (BN / 2));
            if (n >= p.I)
                n = p.I - 1;
            return r < BN / 2 ? n : p.I + n;
        }
        const int n = n_out0 + r;
        return n < p.N ? n : p.N - 1;
    };
    const size_t e_rows = (size_t)e * p.N;
    const char *b_base;
    const char *qs_base = nullptr, *qb_base = nullptr;
    uint32_t b_off[BLOADS];
    uint32_t sb_off[AFF ? BQ : 1];
    if (!AFF) {
        b_base = (const char *)p.B + e_rows * p.K * 2;
#pragma unroll
        for (int i = 0; i < BR; ++i)
            b_off[i] = ((uint32_t)b_row((tid >> 3) + i * 32) * (uint32_t)p.K + chunk * 8) * 2u;
    } else {
        const int groups = p.K / 64;
        b_base = (const char *)p.B + e_rows * (p.K / 2);
        qs_base = (const char *)(p.Bscale + e_rows * groups);
        qb_base = (const char *)(p.Bbias + e_rows * groups);
#pragma unroll
        for (int i = 0; i < BQ; ++i) {
            const int q = tid + i * kThreads;
            const uint32_t row = (uint32_t)b_row(q >> 1);
            b_off[i] = row * (uint32_t)(p.K / 2) + (q & 1) * 16;
            sb_off[i] = row * (uint32_t)groups * 2u;
        }
    }

    uint4 a_reg[AR];
    uint4 b_reg[BLOADS];
    uint32_t sb_reg[AFF ? BQ : 1];

    // staged operand m of a step: A rows first (m < AR), then B rows
    auto load_one = [&](int k0, int m) {
        if (m < AR) {
            a_reg[m] = load16(a_base, a_off[m] + k0 * 2);
        } else if (!AFF) {
            b_reg[m - AR] = load16(b_base, b_off[m - AR] + k0 * 2);
        } else {
            const int i = m - AR;
            b_reg[i] = load16(b_base, b_off[i] + k0 / 2);
            const uint32_t g = sb_off[i] + (k0 / 64) * 2;
            sb_reg[i] = (uint32_t)*(const uint16_t *)(qs_base + g) |
                        ((uint32_t)*(const uint16_t *)(qb_base + g) << 16);
        }
    };
    auto store_one = [&](uint4 *As, int m) {
        uint4 *Bs = As + BM * 8;
        if (m < AR) {
            As[swz((tid >> 3) + m * 32, chunk)] = a_reg[m];
        } else if (!AFF) {
            Bs[swz((tid >> 3) + (m - AR) * 32, chunk)] = b_reg[m - AR];
        } else {
            // 32 codes (half a group of 64) -> bf16 of scale * q + bias
            const int i = m - AR;
            const int q = tid + i * kThreads;
            const int r = q >> 1, half = q & 1;
            const float sc = bf16_to_f32(sb_reg[i] & 0xffffu);
            const float bi = bf16_to_f32(sb_reg[i] >> 16);
            const uint32_t words[4] = {b_reg[i].x, b_reg[i].y, b_reg[i].z, b_reg[i].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t packed[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float lo = __builtin_fmaf(sc, (float)((words[w] >> (8 * c)) & 15u), bi);
                    const float hi = __builtin_fmaf(sc, (float)((words[w] >> (8 * c + 4)) & 15u), bi);
                    packed[c] = pack_bf16x2(lo, hi);
                }
                Bs[swz(r, half * 4 + w)] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
            }
        }
    };
    auto load_step = [&](int k0) {
#pragma unroll
        for (int m = 0; m < AR + BLOADS; ++m)
            load_one(k0, m);
    };
    auto store_step = [&](uint4 *As) {
#pragma unroll
        for (int m = 0; m < AR + BLOADS; ++m)
            store_one(As, m);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    // LDS slot of this lane's fragment piece for each sub-step; the tiles of
    // a wave sit 32 rows apart, which keeps the swizzle and adds 256 slots
    const int a_tile_row = wm * (BM / 2);
    const int b_row0 = gated(MODE) ? wn * (BN / 4) : wn * (BN / 2);
    int b_tile_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (gated(MODE))
            b_tile_off[j] = (j < TN / 2) ? j * 32 : BN / 2 + (j - TN / 2) * 32;
        else
            b_tile_off[j] = j * 32;
        b_tile_off[j] *= 8;
    }
    int a_slot[kBK / 16], b_slot[kBK / 16];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        a_slot[kk] = swz(a_tile_row + (lane & 31), ch);
        b_slot[kk] = BM * 8 + swz(b_row0 + (lane & 31), ch);
    }

    const int KT = p.K / kBK;
    constexpr int NQ = TM * TN;            // MFMAs per sub-step
    constexpr int NF = TM + TN;            // fragment reads per sub-step
    constexpr int NL = AR + BLOADS;        // staged loads (and stores) per step
    bf16x8 af[2][TM], bfr[2][TN];
    auto read_frag = [&](const uint4 *S, int slot, int kk, int m) {
        if (m < TM)
            af[slot][m] = __builtin_bit_cast(bf16x8, S[a_slot[kk] + m * 256]);
        else
            bfr[slot][m - TM] = __builtin_bit_cast(bf16x8, S[b_slot[kk] + b_tile_off[m - TM]]);
    };
    auto mfma = [&](int slot, int q) {
        const int i = q / TN, j = q % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j],
                                                           0, 0, 0);
    };

    // prologue: step 0 staged and stored, step 1 loads in flight, the first
    // fragments read
    load_step(0);
    store_step(smem);
    __syncthreads();
    load_step((KT > 1 ? 1 : 0) * kBK);
#pragma unroll
    for (int m = 0; m < NF; ++m)
        read_frag(smem, 0, 0, m);

    for (int kt = 0; kt < KT; ++kt) {
        const uint4 *S = smem + (kt & 1) * STAGE;
        uint4 *N = smem + ((kt + 1) & 1) * STAGE;
        const int k2 = (kt + 2 < KT ? kt + 2 : KT - 1) * kBK;
        fence();
        // sub-steps 0 and 1
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                mfma(kk & 1, q);
#pragma unroll
                for (int m = q * NF / NQ; m < (q + 1) * NF / NQ; ++m)
                    read_frag(S, (kk + 1) & 1, kk + 1, m);
                fence();
            }
        }
        // sub-step 2: fragments of sub-step 3, then the staged operands of
        // step kt + 1 into the idle buffer
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            mfma(0, q);
#pragma unroll
            for (int m = q * NF / NQ; m < (q + 1) * NF / NQ; ++m)
                read_frag(S, 1, 3, m);
#pragma unroll
            for (int m = q * NL / NQ; m < (q + 1) * NL / NQ; ++m)
                store_one(N, m);
            fence();
        }
        __syncthreads();
        fence();
        // sub-step 3: first fragments of step kt + 1, loads of step kt + 2
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            mfma(1, q);
#pragma unroll
            for (int m = q * NF / NQ; m < (q + 1) * NF / NQ; ++m)
                read_frag(N, 0, 0, m);
#pragma unroll
            for (int m = q * NL / NQ; m < (q + 1) * NL / NQ; ++m)
                load_one(k2, m);
            fence();
        }
    }
    __syncthreads();

    // ---- epilogue. acc[i][j][r] holds row (8*(r/4) + 4*(lane/32) + r%4) and
    // column (lane % 32) of the 32x32 tile (i, j).
    const int col = lane & 31;
    const int rsub = 4 * (lane >> 5);
    if (MODE == kDown) {
        float *y = (float *)p.C;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n_out0 + wn * (BN / 2) + j * 32 + col;
            if (n >= p.N)
                continue;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int orow = s_out_row[a_tile_row + i * 32 + 8 * (r >> 2) + rsub + (r & 3)];
                    if (orow >= 0)
                        y[(size_t)orow * p.ldc + n] = acc[i][j][r];
                }
        }
        return;
    }
    // bf16 h: each wave transposes its (BM/2) x CW block through LDS (the
    // operand buffers are idle after the last barrier) so the global stores
    // are whole 16-byte row pieces
    constexpr int CW = gated(MODE) ? BN / 4 : BN / 2;   // output columns per wave
    constexpr int CT = CW / 32;                              // 32-col tiles per wave
    uint16_t *hs = (uint16_t *)smem + (size_t)wave * (BM / 2) * CW;
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = i * 32 + 8 * (r >> 2) + rsub + (r & 3);
                constexpr bool LIM = MODE == kGateUpLimit;
                const float v = gated(MODE)
                                    ? swiglu<LIM>(acc[i][j][r], acc[i][j + TN / 2][r], p.limit)
                                    : relu_sq(acc[i][j][r]);
                hs[row * CW + j * 32 + col] = (uint16_t)f32_to_bf16(v);
            }
    __syncthreads();
    uint16_t *h = (uint16_t *)p.C;
    const int ncols = gated(MODE) ? p.I : p.N;
    const int wcol0 = n_out0 + wn * CW;
    constexpr int PIECES = (BM / 2) * CW / 8;                // 16-byte pieces per wave
#pragma unroll 4
    for (int q = lane; q < PIECES; q += kWave) {
        const int row = q / (CW / 8), cc = q % (CW / 8);
        const int pos = row0 + a_tile_row + row;
        const int n = wcol0 + cc * 8;
        if (pos < row_end && n < ncols)
            *reinterpret_cast<uint4 *>(h + (size_t)pos * p.ldc + n) =
                *reinterpret_cast<const uint4 *>(hs + row * CW + cc * 8);
    }
}

template <int BM, int MODE, bool AFF>
hipError_t launch_tile(const GemmProblem &p, hipStream_t stream) {
    const int n_cols = gated(MODE) ? p.I : p.N;
    const int n_tile = gated(MODE) ? 128 : 256;
    const int n_tiles = (n_cols + n_tile - 1) / n_tile;
    const int blocks = grid_blocks<BM>(p, n_tiles);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_gemm<BM, MODE, AFF>), dim3(blocks), dim3(kThreads), 0, stream, p,
                       n_tiles);
    return hipGetLastError();
}

template <int MODE, bool AFF>
hipError_t launch_mode(const GemmProblem &p, hipStream_t stream) {
    // segments of a few hundred rows or more take 256-row tiles
    int segs = 1;
    if (p.offsets != nullptr)
        segs = p.E < p.max_rows ? p.E : p.max_rows;
    const int rows = p.offsets != nullptr ? p.max_rows : p.rows;
    const int avg = segs > 0 ? rows / segs : 0;
    if (avg >= 192)
        return launch_tile<256, MODE, AFF>(p, stream);
    return launch_tile<128, MODE, AFF>(p, stream);
}

// k_dequant: the 4-bit weights of the experts with rows, decoded once to
// bf16 for the direct-to-LDS grouped kernel (prompt-sized batches: the
// decoded rows are then read by every m-tile of the expert from L2 or HBM,
// instead of being decoded again in each tile's loads). A code word holds 8
// weights (nibble j at bits 4 j); the decode is the same as the staged
// kernel's, so both paths multiply the same bf16 weights. The workgroups
// share the (expert, chunk) items; each thread decodes 4 words per item.
constexpr int kDqWords = 4;

__global__ __launch_bounds__(kThreads) void k_dequant(GemmProblem p, uint16_t *__restrict__ out) {
    __shared__ int s_list[256];
    __shared__ int s_cnt[kThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // the experts with rows, in expert order
    const bool busy = tid < p.E && p.offsets[tid + 1] > p.offsets[tid];
    const uint64_t m = __ballot(busy);
    if (lane == 0)
        s_cnt[wave] = __popcll(m);
    __syncthreads();
    int rank = __popcll(m & ((1ull << lane) - 1ull)), nb = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
        rank += w < wave ? s_cnt[w] : 0;
        nb += s_cnt[w];
    }
    if (busy)
        s_list[rank] = tid;
    __syncthreads();
    const int K8 = p.K / 8, G = p.K / 64;
    const size_t words = (size_t)p.N * K8;                 // code words per expert
    const size_t per_item = (size_t)kThreads * kDqWords;
    const size_t chunks = (words + per_item - 1) / per_item;
    const uint32_t *codes = (const uint32_t *)p.B;
    for (size_t item = blockIdx.x; item < (size_t)nb * chunks; item += gridDim.x) {
        const int y = (int)(item / chunks);
        const size_t w0 = (item % chunks) * per_item;
        const int e = s_list[y];
#pragma unroll
        for (int j = 0; j < kDqWords; ++j) {
            const size_t w = w0 + (size_t)j * kThreads + tid;
            if (w >= words)
                break;
            const size_t n = w / K8, c8 = w % K8;
            const uint32_t code = codes[(size_t)e * words + w];
            const size_t g = ((size_t)e * p.N + n) * G + c8 / 8;
            const float sc = bf16_to_f32(p.Bscale[g]);
            const float bi = bf16_to_f32(p.Bbias[g]);
            uint32_t packed[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float lo = __builtin_fmaf(sc, (float)((code >> (8 * c)) & 15u), bi);
                const float hi = __builtin_fmaf(sc, (float)((code >> (8 * c + 4)) & 15u), bi);
                packed[c] = pack_bf16x2(lo, hi);
            }
            *reinterpret_cast<uint4 *>(out + ((size_t)y * p.N + n) * p.K + c8 * 8) =
                make_uint4(packed[0], packed[1], packed[2], packed[3]);
        }
    }
}

// Block-FP8 weights of the experts with rows, decoded to bf16 in expert
// order (b_compact), like k_dequant: OCP E4M3 codes (sign, 4 exponent bits
// with bias 7, 3 mantissa bits; exponent 0 holds m * 2^-9; S.1111.111 is
// NaN), each times the fp32 scale of its 128 x 128 block, rounded once to
// bf16. A thread decodes 16 consecutive codes of a row (one 16-byte load,
// one scale) per item.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const uint32_t sign = (b & 0x80u) << 24;
    float v = e != 0 ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                     : (float)m * 0x1p-9f;
    v = (e == 15u && m == 7u) ? __builtin_nanf("") : v;
    return __uint_as_float(__float_as_uint(v) | sign);
}

__global__ __launch_bounds__(kThreads) void k_dequant_fp8(GemmProblem p,
                                                          uint16_t *__restrict__ out) {
    __shared__ int s_list[256];
    __shared__ int s_cnt[kThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool busy = tid < p.E && p.offsets[tid + 1] > p.offsets[tid];
    const uint64_t m = __ballot(busy);
    if (lane == 0)
        s_cnt[wave] = __popcll(m);
    __syncthreads();
    int rank = __popcll(m & ((1ull << lane) - 1ull)), nb = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
        rank += w < wave ? s_cnt[w] : 0;
        nb += s_cnt[w];
    }
    if (busy)
        s_list[rank] = tid;
    __syncthreads();
    const int K16 = p.K / 16, KB = p.K / 128, NB = p.N / 128;
    const size_t pieces = (size_t)p.N * K16;               // 16-code pieces per expert
    const size_t chunks = (pieces + kThreads - 1) / kThreads;
    const uint8_t *codes = (const uint8_t *)p.B;
    const float *scales = (const float *)p.Bscale;
    for (size_t item = blockIdx.x; item < (size_t)nb * chunks; item += gridDim.x) {
        const int y = (int)(item / chunks);
        const size_t q = (item % chunks) * kThreads + tid;
        if (q >= pieces)
            continue;
        const int e = s_list[y];
        const size_t n = q / K16, c16 = q % K16;
        const uint4 v = *reinterpret_cast<const uint4 *>(codes + ((size_t)e * p.N + n) * p.K +
                                                         c16 * 16);
        const float sc = scales[((size_t)e * NB + n / 128) * KB + c16 / 8];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            packed[2 * i] = pack_bf16x2(e4m3_to_f32(w[i] & 0xffu) * sc,
                                        e4m3_to_f32((w[i] >> 8) & 0xffu) * sc);
            packed[2 * i + 1] = pack_bf16x2(e4m3_to_f32((w[i] >> 16) & 0xffu) * sc,
                                            e4m3_to_f32(w[i] >> 24) * sc);
        }
        uint4 *o = reinterpret_cast<uint4 *>(out + ((size_t)y * p.N + n) * p.K + c16 * 16);
        o[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        o[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    }
}

}  // namespace

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream) {
    if (grouped_supported(p))
        return launch_grouped(p, stream);        // FP8 included (its own tiles)
    if (p.E2 > 0 || p.Bglobal != nullptr || p.nvfp4 || p.mxfp4)
        return hipErrorInvalidValue;             // shared segments, global scales: the
                                                 // persistent kernel only
    if (p.fp8)
        return hipErrorInvalidValue;             // otherwise decoded by launch_dequant first
    if (p.affine4) {
        switch (p.mode) {
        case kGateUp: return launch_mode<kGateUp, true>(p, stream);
        case kGateUpLimit: return launch_mode<kGateUpLimit, true>(p, stream);
        case kUpRelu2: return launch_mode<kUpRelu2, true>(p, stream);
        default: return launch_mode<kDown, true>(p, stream);
        }
    }
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp, false>(p, stream);
    case kGateUpLimit: return launch_mode<kGateUpLimit, false>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2, false>(p, stream);
    default: return launch_mode<kDown, false>(p, stream);
    }
}

hipError_t launch_dequant(const GemmProblem &p, uint16_t *out, hipStream_t stream) {
    if (p.fp8) {
        if (p.offsets == nullptr || p.E > 256 || p.K % 128 != 0 || p.N % 128 != 0)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_dequant_fp8, dim3(1024), dim3(kThreads), 0, stream, p, out);
        return hipGetLastError();
    }
    if (!p.affine4 || p.offsets == nullptr || p.E > 256 || p.K % 64 != 0)
        return hipErrorInvalidValue;
    // a few workgroups per CU share the items
    hipLaunchKernelGGL(k_dequant, dim3(1024), dim3(kThreads), 0, stream, p, out);
    return hipGetLastError();
}

}  // namespace moe
