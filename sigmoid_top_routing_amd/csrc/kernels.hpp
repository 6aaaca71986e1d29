// kernels.hpp -- host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Plan outputs the router may build itself (all NULL: it does not).
struct PlanOut {
    int32_t *counts;    // [E]
    int32_t *offsets;   // [E+1]
    int32_t *sorted;    // [T*k]
    int32_t *slot_of;   // [T*k]
};
constexpr int kFusedPlanMaxA = 1024;

// Router + top-k: a logits launch and a top-k launch. z_scratch holds the
// [T][E] fp32 logits between them, or for batches of at most 8 tokens and
// 32 experts the [H/64][T][E] partial logits of the slices
// (route_scratch_bytes). When `plan` is given and one top-k workgroup covers
// every token (decode-sized batches), the top-k launch also writes the plan
// and *plan_done is set; otherwise the caller runs launch_plan.
size_t route_scratch_bytes(int T, int H, int E);
// softmax: 0 sigmoid scores, 1 the softmax of each token's logits.
hipError_t launch_route(const uint16_t *x, const float *Wr, const float *bias, int T, int H, int E,
                        int k, int softmax, int norm_topk, float eps, int32_t *ids,
                        float *weights, float *z_scratch, PlanOut plan, bool *plan_done,
                        hipStream_t stream);

// Plan scratch: per-chunk expert counts, plan_chunks(A) x E int32.
int plan_chunk_size(int A);
int plan_chunks(int A);
// seg_offsets (optional): [E + shared_segs + 1], the offsets followed by
// shared_segs segments of T rows each (the shared expert as plan segments,
// all T tokens in each); sorted then holds A + shared_segs * T entries, the
// shared positions A + v T + t holding t * k (token t through the gather).
hipError_t launch_plan(const int32_t *ids, int A, int E, int32_t *counts, int32_t *offsets,
                       int32_t *sorted, int32_t *slot_of, int32_t *fault, int32_t *chunk_counts,
                       hipStream_t stream, int32_t *seg_offsets = nullptr, int shared_segs = 0,
                       int T = 0);

// Grouped GEMM over expert segments.
// kGateUpLimit: kGateUp with the SwiGLU inputs clamped at GemmProblem::limit.
enum GemmMode { kGateUp = 0, kUpRelu2 = 1, kDown = 2, kGateUpLimit = 3 };
constexpr bool gated(int mode) { return mode == kGateUp || mode == kGateUpLimit; }

// The weighted combine of launch_combine, as launch_down_combine takes it.
struct CombineArgs {
    const int32_t *slot;      // slot_of [T*k]: the plan position of assignment t*k + j
    const float *w;           // weights [T*k]
    const float *shared;      // NULL or shared_terms rows of [T][H], T*H apart
    int shared_terms;
    int T;
    int k;
    float rsf;                // routed scale
    int fold;                 // the routed scale folded into each weight
    void *out;                // [T][H], bf16 or fp32
    int out_f32;
};

struct GemmProblem {
    int mode;                 // GemmMode
    int affine4;              // B is 4-bit affine (codes + bf16 scale / bias, group 64)
    int fp8;                  // B is block-FP8 e4m3 (bytes + fp32 scale per 128 x 128 block):
                              // the persistent kernel (grouped_supported), the stream
                              // (stream_supported) or launch_dequant reads it
    int nvfp4;                // B is NVFP4: e2m1 codes [E][N][K/2] (low nibble first), an
                              // e4m3 scale byte per 16 inputs [E][N][K/16]: the stream or
                              // launch_dequant reads it
    int mxfp4;                // B is MXFP4: the same codes, an E8M0 scale byte per 32
                              // inputs [E][N][K/32] (2^(b-127), 0xFF NaN): the stream or
                              // launch_dequant reads it
    const uint16_t *A;        // bf16 rows, lda elements apart
    int lda;
    int a_blocked;            // A in row blocks (the persistent kernel's output with
                              // c_blocked): rows in groups of 16, each group's K-slices of
                              // 32 columns 1 KB apiece; not gathered
    int c_blocked;            // kGateUp / kUpRelu2 on the persistent kernel: C (bf16) in those
                              // row blocks, for a down projection with a_blocked
    const int32_t *gather;    // A row of position p = gather[p] / gather_div (NULL: row p)
    int gather_div;
    const int32_t *offsets;   // [E+1] segment bounds (NULL: one segment [0, rows))
    int rows;                 // rows when offsets == NULL
    int E;
    int max_rows;             // bound on offsets[E] (sizes the grid)
    const void *B;            // [E][N][K] bf16, or uint32 codes [E][N][K/8]
    const void *Btiles;       // bf16 or FP8 B's tile-packed copy (launch_pack_tiles) or
                              // NULL; the persistent kernel's expert tiles read it instead of B
    const uint16_t *Bscale;   // [E][N][K/64] (affine-4); fp32 [E][N/128][K/128] (fp8)
    const uint16_t *Bbias;
    int N;                    // rows of B per expert
    int K;
    int I;                    // kGateUp: gate rows are 0..I-1, up rows I..2I-1
    void *C;                  // kGateUp / kUpRelu2: bf16 [rows][ldc]; kDown: fp32 [*][ldc]
    int ldc;
    const int32_t *scatter;   // kDown: output row of position p = scatter[p] (NULL: row p)
    int b_compact;            // B holds only the experts with rows, in expert order
    float limit;              // kGateUpLimit: the SwiGLU input limit L > 0
    // Segments E .. E + E2 - 1 after the experts (the shared expert as plan
    // segments; bf16, the persistent kernel only): segment E + v reads its
    // weights at B2 + v * b2_vstride elements, rows b2_ld elements apart,
    // and (gated) its up rows b2_up rows after its gate rows.
    const uint16_t *B2;
    int E2;
    int b2_ld;
    int b2_up;
    long long b2_vstride;
    // Per-expert fp32 scale of the sums (NVFP4's global scale; NULL: none),
    // applied before the epilogue, indexed by expert (not by compact rank);
    // the persistent kernel and the quantized stream apply it.
    const float *Bglobal;
};

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream);

// The 4-bit (p.affine4) or block-FP8 (p.fp8) weights of p's experts that
// have rows (offsets set), decoded once to bf16 (scale * q + bias or scale
// * e4m3 value, in fp32, rounded to nearest even) into out: [experts with
// rows][N][K], in expert order (b_compact).
hipError_t launch_dequant(const GemmProblem &p, uint16_t *out, hipStream_t stream);

// The persistent direct-to-LDS kernel (bf16 weights, K a multiple of 32 and
// at least 128); launch_gemm routes the problems it supports there.
bool grouped_supported(const GemmProblem &p);
hipError_t launch_grouped(const GemmProblem &p, hipStream_t stream);
// The tile-packed copy of a weight tensor w [E][N][K] of bf16 (esz 2) or FP8
// codes (esz 1) (K a multiple of 32; gate_up: N = 2 I, gate rows first) and
// its size in bytes: for each expert and n-tile (256 weight rows; SwiGLU:
// 128 gate rows and their 128 up rows), K / 32 slices of 16 or 8 KB in the
// order the persistent kernel's stages hold them.
size_t pack_tiles_bytes(int E, int N, int K, int I, bool gate_up, int esz);
hipError_t launch_pack_tiles(const void *w, void *tiles, int E, int N, int K, int I, bool gate_up,
                             int esz, hipStream_t stream);
// Its block-FP8 form (grouped_gemm_f8.hip); launch_grouped calls it.
hipError_t launch_grouped_f8(const GemmProblem &p, hipStream_t stream);
// NVFP4 / MXFP4 weights on the MFMA tiles (grouped_gemm_f4.hip)
hipError_t launch_grouped_f4(const GemmProblem &p, hipStream_t stream);

// The same problem in the weight-streaming (decode) form: few A rows per
// expert, every touched weight row read once, v_dot2 accumulation.
// Largest K the quantized decode form takes (4 steps of 16 code bytes per
// lane: 8192 4-bit weights, 4096 FP8 weights).
constexpr int kStreamMaxKAffine4 = 8192;
constexpr int kStreamMaxKFp8 = 4096;
constexpr int kStreamMaxKNvfp4 = 8192;
constexpr int kStreamMaxKMxfp4 = 8192;
bool stream_supported(const GemmProblem &p);
hipError_t launch_stream(const GemmProblem &p, hipStream_t stream);
// The decode form's bf16 down projection (kDown, offsets set, at most 32
// plan positions, K <= 2048) with the weighted combine of launch_combine in
// the same launch: out is written, y (p.C) is not.
bool down_combine_supported(const GemmProblem &p, int T, int k);
hipError_t launch_down_combine(const GemmProblem &p, const CombineArgs &c, hipStream_t stream);

// Fused residual add + RMSNorm of T rows of H (a multiple of 64, at most
// kNormMaxH): residual_out = bf16(h + residual), x = bf16(r gamma / rms).
// h and residual_out may be NULL; residual_out may equal residual.
constexpr int kNormMaxH = 8192;
hipError_t launch_add_rmsnorm(const uint16_t *h, const uint16_t *residual, const uint16_t *gamma,
                              int T, int H, float eps, uint16_t *residual_out, uint16_t *x,
                              hipStream_t stream);

// out[t] = routed_scale * sum_j weights[t,j] y_seg[slot_of[t*k+j]] + s[t], or with
// fold, sum_j (routed_scale * weights[t,j]) y_seg[slot_of[t*k+j]] (no shared term);
// s[t] = shared[t] + shared[T + t] + ... over shared_terms rows T*H apart (v
// ascending; one term: the shared output itself).
hipError_t launch_combine(const float *y_seg, const int32_t *slot_of, const float *weights,
                          const float *shared, int shared_terms, int T, int H, int k,
                          float routed_scale, bool fold, void *out, int out_f32,
                          hipStream_t stream);

}  // namespace moe
