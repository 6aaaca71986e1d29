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
hipError_t launch_plan(const int32_t *ids, int A, int E, int32_t *counts, int32_t *offsets,
                       int32_t *sorted, int32_t *slot_of, int32_t *fault, int32_t *chunk_counts,
                       hipStream_t stream);

// Grouped GEMM over expert segments.
// kGateUpLimit: kGateUp with the SwiGLU inputs clamped at GemmProblem::limit.
enum GemmMode { kGateUp = 0, kUpRelu2 = 1, kDown = 2, kGateUpLimit = 3 };
constexpr bool gated(int mode) { return mode == kGateUp || mode == kGateUpLimit; }

struct GemmProblem {
    int mode;                 // GemmMode
    int affine4;              // B is 4-bit affine (codes + bf16 scale / bias, group 64)
    int fp8;                  // B is block-FP8 e4m3 (bytes + fp32 scale per 128 x 128 block):
                              // only launch_dequant reads it
    const uint16_t *A;        // bf16 rows, lda elements apart
    int lda;
    const int32_t *gather;    // A row of position p = gather[p] / gather_div (NULL: row p)
    int gather_div;
    const int32_t *offsets;   // [E+1] segment bounds (NULL: one segment [0, rows))
    int rows;                 // rows when offsets == NULL
    int E;
    int max_rows;             // bound on offsets[E] (sizes the grid)
    const void *B;            // [E][N][K] bf16, or uint32 codes [E][N][K/8]
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
};

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream);

// The 4-bit (p.affine4) or block-FP8 (p.fp8) weights of p's experts that
// have rows (offsets set), decoded once to bf16 (scale * q + bias, or
// scale * e4m3 value, in fp32, rounded to nearest even) into out:
// [experts with rows][N][K], in expert order (b_compact).
hipError_t launch_dequant(const GemmProblem &p, uint16_t *out, hipStream_t stream);

// The persistent direct-to-LDS kernel (bf16 weights, K a multiple of 32 and
// at least 128); launch_gemm routes the problems it supports there.
bool grouped_supported(const GemmProblem &p);
hipError_t launch_grouped(const GemmProblem &p, hipStream_t stream);

// The same problem in the weight-streaming (decode) form: few A rows per
// expert, every touched weight row read once, v_dot2 accumulation.
bool stream_supported(const GemmProblem &p);
hipError_t launch_stream(const GemmProblem &p, hipStream_t stream);

// Fused residual add + RMSNorm of T rows of H (a multiple of 64, at most
// kNormMaxH): residual_out = bf16(h + residual), x = bf16(r gamma / rms).
// h and residual_out may be NULL; residual_out may equal residual.
constexpr int kNormMaxH = 8192;
hipError_t launch_add_rmsnorm(const uint16_t *h, const uint16_t *residual, const uint16_t *gamma,
                              int T, int H, float eps, uint16_t *residual_out, uint16_t *x,
                              hipStream_t stream);

// out[t] = routed_scale * sum_j weights[t,j] y_seg[slot_of[t*k+j]] + shared[t]
hipError_t launch_combine(const float *y_seg, const int32_t *slot_of, const float *weights,
                          const float *shared, int T, int H, int k, float routed_scale, void *out,
                          int out_f32, hipStream_t stream);

}  // namespace moe
