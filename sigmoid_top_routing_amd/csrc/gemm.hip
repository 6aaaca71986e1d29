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
// Tiling. A workgroup of 4 waves owns a BM x BN tile of one expert and
// walks K in steps of 64. Per step it stages the A rows (gathered through
// the plan: row(p) = gather[p] / gather_div, so x is never permuted in
// memory) and the BN weight rows in LDS, double buffered, with a 16-byte
// XOR swizzle so the MFMA operand reads hit distinct banks. Each wave owns
// a (BM/2) x (BN/2) quarter and issues v_mfma_f32_32x32x16_bf16 over it.
// For kGateUp a tile's BN weight rows are BN/2 gate rows and the BN/2 up
// rows that pair with them, and each wave takes matching gate and up
// columns, so silu(g) * u is formed in registers without an LDS exchange.
// The 4-bit affine form decodes its codes (scale * q + bias, group 64) to
// bf16 on the way into LDS; the MFMA loop is the same.
//
// Tile order. Workgroups are dispatched to the 8 XCDs round robin, so the
// block index is remapped to give each XCD a contiguous run of the logical
// order (n-tile major, m-tile minor): the m-tiles that share a weight tile
// then run on one XCD and share its L2.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 8 + (chunk ^ (row & 7));
}

// Which expert segment and which BM rows of it this workgroup owns.
// Returns false when the m-tile index is past the last real tile.
template <int BM>
__device__ bool locate_tile(const GemmProblem &p, int mt, int *e_out, int *row0, int *row_end) {
    if (p.offsets == nullptr) {
        const int tiles = (p.rows + BM - 1) / BM;
        if (mt >= tiles)
            return false;
        *e_out = 0;
        *row0 = mt * BM;
        *row_end = p.rows;
        return true;
    }
    __shared__ int s_wsum[4];
    __shared__ int s_hit[3];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    int tiles = 0, lo = 0, hi = 0;
    if (tid < p.E) {
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
    for (int w = 0; w < wave; ++w)
        incl += s_wsum[w];
    const int excl = incl - tiles;
    if (tid < p.E && mt >= excl && mt < incl) {
        s_hit[0] = tid;
        s_hit[1] = lo + (mt - excl) * BM;
        s_hit[2] = hi;
    }
    __syncthreads();
    if (s_hit[0] < 0)
        return false;
    *e_out = s_hit[0];
    *row0 = s_hit[1];
    *row_end = s_hit[2];
    return true;
}

template <int BM, int BN, int MODE, bool AFF>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmProblem p, int mt_max) {
    constexpr int TM = BM / 64;          // 32-row MFMA tiles per wave
    constexpr int TN = BN / 64;          // 32-col MFMA tiles per wave
    constexpr int AR = BM / 32;          // A rows staged per thread per step
    constexpr int BR = BN / 32;          // B rows staged per thread per step (bf16)
    constexpr int BQ = BN / 128;         // B half-rows per thread per step (affine-4)
    static_assert(TN % 2 == 0, "gate and up columns come in pairs");

    __shared__ uint4 As[2][BM * 8];
    __shared__ uint4 Bs[2][BN * 8];
    __shared__ int s_out_row[BM];

    // ---- tile
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int L = (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
    const int nt = L / mt_max;
    const int mt = L % mt_max;
    int e, row0, row_end;
    if (!locate_tile<BM>(p, mt, &e, &row0, &row_end))
        return;
    const int n_out0 = nt * (MODE == kGateUp ? BN / 2 : BN);

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

    // ---- A rows this thread stages
    const uint16_t *a_ptr[AR];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
        const int r = (tid >> 3) + i * 32;
        const int pos = row0 + r;
        if (pos < row_end) {
            const int arow = p.gather ? p.gather[pos] / p.gather_div : pos;
            a_ptr[i] = p.A + (size_t)arow * p.lda + chunk * 8;
        } else {
            a_ptr[i] = nullptr;
        }
    }

    // ---- B rows this thread stages
    auto b_row = [&](int r, bool *ok) -> int {
        if (MODE == kGateUp) {
            const int half = BN / 2;
            const int n = n_out0 + (r % half);
            *ok = n < p.I;
            return r < half ? n : p.I + n;
        }
        const int n = n_out0 + r;
        *ok = n < p.N;
        return n;
    };
    const uint16_t *b_ptr[AFF ? 1 : BR];
    const uint32_t *q_ptr[AFF ? BQ : 1];
    const uint16_t *qs_ptr[AFF ? BQ : 1];
    const uint16_t *qb_ptr[AFF ? BQ : 1];
    if (!AFF) {
#pragma unroll
        for (int i = 0; i < BR; ++i) {
            bool ok;
            const int wr = b_row((tid >> 3) + i * 32, &ok);
            b_ptr[i] = ok ? (const uint16_t *)p.B + ((size_t)e * p.N + wr) * p.K + chunk * 8
                          : nullptr;
        }
    } else {
        const int groups = p.K / 64;
#pragma unroll
        for (int i = 0; i < BQ; ++i) {
            const int q = tid + i * kThreads;
            bool ok;
            const int wr = b_row(q >> 1, &ok);
            const size_t row = (size_t)e * p.N + wr;
            q_ptr[i] = ok ? (const uint32_t *)p.B + row * (p.K / 8) + (q & 1) * 4 : nullptr;
            qs_ptr[i] = ok ? p.Bscale + row * groups : nullptr;
            qb_ptr[i] = ok ? p.Bbias + row * groups : nullptr;
        }
    }

    uint4 a_reg[AR];
    uint4 b_reg[AFF ? BQ : BR];
    uint32_t sb_reg[AFF ? BQ : 1];

    auto load_step = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AR; ++i)
            a_reg[i] = a_ptr[i] ? *reinterpret_cast<const uint4 *>(a_ptr[i] + k0)
                                : make_uint4(0, 0, 0, 0);
        if (!AFF) {
#pragma unroll
            for (int i = 0; i < BR; ++i)
                b_reg[i] = b_ptr[i] ? *reinterpret_cast<const uint4 *>(b_ptr[i] + k0)
                                    : make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < BQ; ++i) {
                if (q_ptr[i]) {
                    b_reg[i] = *reinterpret_cast<const uint4 *>(q_ptr[i] + k0 / 8);
                    sb_reg[i] = (uint32_t)qs_ptr[i][k0 / 64] | ((uint32_t)qb_ptr[i][k0 / 64] << 16);
                } else {
                    b_reg[i] = make_uint4(0, 0, 0, 0);
                    sb_reg[i] = 0;   // scale 0, bias 0: a zero row
                }
            }
        }
    };

    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AR; ++i)
            As[buf][swz((tid >> 3) + i * 32, chunk)] = a_reg[i];
        if (!AFF) {
#pragma unroll
            for (int i = 0; i < BR; ++i)
                Bs[buf][swz((tid >> 3) + i * 32, chunk)] = b_reg[i];
        } else {
#pragma unroll
            for (int i = 0; i < BQ; ++i) {
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
                    Bs[buf][swz(r, half * 4 + w)] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
                }
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    // rows of the B tile each of this wave's column tiles reads
    int b_tile_row[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (MODE == kGateUp)
            b_tile_row[j] = (j < TN / 2) ? wn * (BN / 4) + j * 32
                                         : BN / 2 + wn * (BN / 4) + (j - TN / 2) * 32;
        else
            b_tile_row[j] = wn * (BN / 2) + j * 32;
    }
    const int a_tile_row = wm * (BM / 2);

    const int KT = p.K / kBK;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT)
            load_step((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = a_tile_row + i * 32 + (lane & 31);
                af[i] = __builtin_bit_cast(bf16x8, As[buf][swz(r, ch)]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = b_tile_row[j] + (lane & 31);
                bfr[j] = __builtin_bit_cast(bf16x8, Bs[buf][swz(r, ch)]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                       0, 0, 0);
        }
        if (kt + 1 < KT)
            store_step(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue. acc[i][j][r] holds row (8*(r/4) + 4*(lane/32) + r%4) and
    // column (lane % 32) of the 32x32 tile (i, j).
    const int col = lane & 31;
    const int rsub = 4 * (lane >> 5);
    if (MODE == kGateUp) {
        uint16_t *h = (uint16_t *)p.C;
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
            const int n = n_out0 + wn * (BN / 4) + j * 32 + col;
            if (n >= p.I)
                continue;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int pos = row0 + a_tile_row + i * 32 + 8 * (r >> 2) + rsub + (r & 3);
                    if (pos < row_end)
                        h[(size_t)pos * p.ldc + n] =
                            (uint16_t)f32_to_bf16(silu_mul(acc[i][j][r], acc[i][j + TN / 2][r]));
                }
        }
    } else if (MODE == kUpRelu2) {
        uint16_t *h = (uint16_t *)p.C;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n_out0 + wn * (BN / 2) + j * 32 + col;
            if (n >= p.N)
                continue;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int pos = row0 + a_tile_row + i * 32 + 8 * (r >> 2) + rsub + (r & 3);
                    if (pos < row_end)
                        h[(size_t)pos * p.ldc + n] = (uint16_t)f32_to_bf16(relu_sq(acc[i][j][r]));
                }
        }
    } else {
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
    }
}

template <int BM, int BN, int MODE, bool AFF>
hipError_t launch_tile(const GemmProblem &p, hipStream_t stream) {
    int mt_max;
    if (p.offsets == nullptr) {
        mt_max = (p.rows + BM - 1) / BM;
    } else {
        const int nonempty = p.E < p.max_rows ? p.E : p.max_rows;
        mt_max = (p.max_rows + BM - 1) / BM + nonempty;
    }
    const int n_cols = MODE == kGateUp ? p.I : p.N;
    const int n_tile = MODE == kGateUp ? BN / 2 : BN;
    const int nt = (n_cols + n_tile - 1) / n_tile;
    int blocks = mt_max * nt;
    if (blocks == 0)
        return hipSuccess;
    // round the grid up to whole XCD rounds; mt_max absorbs the padding
    while ((mt_max * nt) % kXcds)
        ++mt_max;
    blocks = mt_max * nt;
    hipLaunchKernelGGL((k_gemm<BM, BN, MODE, AFF>), dim3(blocks), dim3(kThreads), 0, stream, p,
                       mt_max);
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
        return launch_tile<256, 256, MODE, AFF>(p, stream);
    return launch_tile<128, 256, MODE, AFF>(p, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream) {
    if (p.affine4) {
        switch (p.mode) {
        case kGateUp: return launch_mode<kGateUp, true>(p, stream);
        case kUpRelu2: return launch_mode<kUpRelu2, true>(p, stream);
        default: return launch_mode<kDown, true>(p, stream);
        }
    }
    switch (p.mode) {
    case kGateUp: return launch_mode<kGateUp, false>(p, stream);
    case kUpRelu2: return launch_mode<kUpRelu2, false>(p, stream);
    default: return launch_mode<kDown, false>(p, stream);
    }
}

}  // namespace moe
