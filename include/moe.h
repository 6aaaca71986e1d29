/*
 * moe.h -- C ABI of the sigmoid top-k routed mixture-of-experts block on
 * AMD Instinct MI355X (gfx950).
 *
 * The block, for a token row x_t (H inputs):
 *   z[e]  = p_0 + p_1 + ... + p_{H/64-1}   fp32, added in ascending j from +0, where
 *   p_j   = x[t,64j] Wr[e,64j] + ... + x[t,64j+63] Wr[e,64j+63]
 *                                          fp32, one fmaf per term, h ascending, from +0
 *           (the router's K slices are 64 wide and fixed by H alone; TensorFold
 *           issue #548, the Nemotron score top-k that adds the router's K
 *           slices itself, and the kernel rule that slices come from the
 *           weight's shape, so a row's bits do not depend on the batch)
 *   s[e]  = 1 / (1 + exp(-z[e]))           fp32 (own exp, correctly rounded division)
 *           or softmax: q[e] = exp(z[e] - max z) (0 below -87), s[e] = q[e] / sum q,
 *           the sum from +0 in expert order (score_fn)
 *   ids   = the k experts of largest s[e] + bias[e]; the bias only selects
 *   w_j   = s[ids_j] / (sum_j s[ids_j] + norm_eps)   (or s[ids_j] when norm_topk == 0)
 *   y_j   = W_down[e] act(W_up[e] x_t),  e = ids_j
 *             SwiGLU: W_up = gate_up (E, 2I, H), gate rows first,
 *                     act = silu(min(gate, L)) * clamp(up, -L, L)
 *                     (swiglu_limit L; no clamp when L == 0)
 *             relu^2: W_up = up (E, I, H), act = (up < 0 ? 0 : up)^2
 *   out_t = routed_scale * sum_j w_j y_j + shared_t
 *   shared_t = W_sd act(W_su x_t), added unscaled (optional)
 *   (or, with fold_routed_scale and no shared expert,
 *    out_t = sum_j (routed_scale w_j) y_j)
 * Sources: TileGym PR #187, "Weight layout and routing" (gate_up layout,
 * sigmoid routing, bias used only for selection, sum + 1e-6, then the routed
 * scaling factor); TensorFold PR #1492, "What" and "Verification" (fp32
 * router weights with expert bias and eps 1e-6; an all-NaN row must not
 * pick one expert twice); vllm.cpp PR #684, "The seam decision" and its W2
 * commit (relu^2 expert; the routed scale multiplies the finished routed
 * sum, the shared output is added untouched; outputs are f32 or bf16 only);
 * TensorFold issue #548 (one grouped-MoE layer: routing plan plus
 * per-format experts behind one call, decode rows and prompt rows; the
 * softmax router family in its consolidation proposal; GLM's swiglu_limit
 * in its table of untested expert paths, where about 16 % of gate and 33 %
 * of up pre-activations clamp at limit 10: the gate on one side, up on
 * both).
 *
 * Conventions for every entry point:
 *  - Tensors are row-major and live in device memory owned by the caller.
 *    bf16 tensors are passed as uint16_t bit patterns. Every tensor pointer
 *    must be 16-byte aligned.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream). The library never allocates, frees or
 *    synchronises device memory; scratch comes from the caller's workspace.
 *  - Arguments are checked on the host before anything is enqueued. On an
 *    error nothing is enqueued, the return value is a negative moe_status
 *    and moe_last_error() names the argument and what was expected.
 *  - Results are deterministic: the same inputs give the same bytes, on any
 *    stream, whatever else runs beside them.
 *  - Calls are re-entrant; two calls that share a workspace must not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_E_NULL = -1,        /* a required pointer is NULL */
    MOE_E_SHAPE = -2,       /* a size is out of range or not a multiple it must be */
    MOE_E_ALIGN = -3,       /* a tensor pointer is not 16-byte aligned */
    MOE_E_UNSUPPORTED = -4, /* an option value this build does not implement */
    MOE_E_WORKSPACE = -5,   /* workspace smaller than moe_workspace_bytes() */
    MOE_E_HIP = -6          /* the HIP runtime refused a launch */
} moe_status;

typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 } moe_act;
typedef enum {
    MOE_W_BF16 = 0,
    MOE_W_AFFINE4 = 1,
    MOE_W_FP8 = 2,
    MOE_W_NVFP4 = 3,
    MOE_W_MXFP4 = 4
} moe_wfmt;
typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_out;
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score;

/* Shape and options of one layer call. Limits: T >= 0; 1 <= E <= 256;
 * 1 <= k <= min(E, 8); H, I and I_shared multiples of 64 (I_shared may be
 * 0: no shared expert); group == 64 for MOE_W_AFFINE4 (0 otherwise). */
typedef struct {
    int32_t T;            /* tokens */
    int32_t H;            /* hidden size (router and expert input, block output) */
    int32_t I;            /* expert intermediate size */
    int32_t E;            /* experts */
    int32_t k;            /* experts per token */
    int32_t act;          /* moe_act; the shared expert uses the same activation */
    int32_t wfmt;         /* moe_wfmt of the routed experts */
    int32_t group;        /* 4-bit group size along the input dimension (64) */
    int32_t norm_topk;    /* 1: w = s / (sum s + norm_eps); 0: w = s */
    float norm_eps;       /* 1e-6 on LFM2-MoE and Nemotron-H */
    float routed_scale;   /* applied once, to the routed sum only */
    int32_t I_shared;     /* shared-expert intermediate size, 0 = none */
    int32_t out_dtype;    /* moe_out */
    int32_t score_fn;     /* moe_score: router scores (the bias, if any, still only selects) */
    float swiglu_limit;   /* 0: none; L > 0 (SwiGLU only, routed and shared experts):
                             gate capped at L, up clamped to [-L, L], NaN kept */
    int32_t fold_routed_scale; /* 0: routed_scale multiplies the finished routed sum
                             (the Nemotron-H order); 1: Laguna's fold, routed_scale
                             multiplies each expert weight inside the sum, the
                             fp32 product routed_scale * w_j taken once per term
                             (vllm.cpp PR #684, the review-repairs commit: equal in
                             exact arithmetic, different fp32 bits; legal only
                             without a shared expert, so I_shared must be 0) */
    int32_t row_invariant; /* 0: decode-sized batches (T * k <= 2 E) take the
                             weight-streaming form, whose fp32 sums differ from the
                             MFMA tiles' in the last bits; 1: every batch takes the
                             MFMA tiles (4-bit experts decoded to bf16 first;
                             block-FP8, NVFP4 and MXFP4 codes on their own
                             tiles), so a
                             token's output bits do not depend on how many tokens
                             share the call (TensorFold issue #548, the kernel
                             registry's family rule), at the tiles' cost for decode
                             batches. Holds while every projection fits the tiles:
                             T*k*max(H, I)*2 < 2^31 and, for block-FP8, H and I at
                             most 8192. */
} moe_dims;

/* Weights of one layer (device pointers).
 *  router_w    fp32 [E, H]
 *  expert_bias fp32 [E] or NULL (selection only, never in the weights)
 *  w_up        SwiGLU: [E, 2I, H], gate rows 0..I-1 then up rows I..2I-1;
 *              relu^2: [E, I, H]
 *  w_down      [E, H, I]
 *  For MOE_W_BF16 w_up / w_down are bf16 and the *_scales / *_biases are
 *  unused. For MOE_W_AFFINE4 they are uint32 words of 4-bit codes
 *  ([E, N, K/8]: element c of a row is bits 4*(c%8) of word c/8), and
 *  w_*_scales / w_*_biases are bf16 [E, N, K/64]; the weight is
 *  scale * code + bias (MLX 4-bit affine, group 64; TensorFold PR #1492
 *  "What").
 *  For MOE_W_FP8 (block-FP8; TensorFold issue #548, the block-FP8 experts of
 *  its CUDA branches) they are uint8 OCP E4M3 codes [E, N, K] (sign, 4
 *  exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 *  NaN; largest 448), w_*_scales are fp32 [E, N/128, K/128], one per
 *  128 x 128 block, the weight is scale * value, and w_*_biases are unused.
 *  H and I must then be multiples of 128, and every scale finite and
 *  non-zero (as an absmax quantizer's scales are; a zero or non-finite scale
 *  gives undefined outputs). The codes are read at one byte per weight and
 *  converted exactly to bf16 (every E4M3 value is a bf16 value); the block
 *  scales multiply fp32 sums: decode-sized batches stream the codes and
 *  scale each lane's partial over 16 inputs of one block, larger ones run
 *  the MFMA tiles, whose running sums are rescaled at each 128-wide K-block
 *  boundary. With H or I above 8192 a prompt-sized batch decodes the experts
 *  with rows to bf16 (scale * value rounded) in the workspace first.
 *  For MOE_W_NVFP4 (ModelOpt NVFP4; TensorFold issue #548, the core/quant
 *  split: uint8 [N, K/2], an e4m3 scale every 16 inputs, a global scale)
 *  they are uint8 [E, N, K/2], two FP4 E2M1 codes per byte (sign bit 3,
 *  exponent bits 2..1 with bias 1, mantissa bit 0: magnitudes 0, 0.5, 1,
 *  1.5, 2, 3, 4, 6), element c of a row in byte c/2, low nibble first (this
 *  library's stated packing); w_*_scales are OCP E4M3 bytes [E, N, K/16],
 *  one per 16 inputs; w_up_global / w_down_global are fp32 [E], one per
 *  expert matrix (the fused gate_up matrix has one); the weight is
 *  e2m1 * scale * global, and w_*_biases are unused. Every e2m1 * scale
 *  product is exact in bf16: decode-sized batches stream the codes and
 *  scale each 16-input partial in fp32; larger ones (and every batch with
 *  row_invariant) read the codes on the MFMA tiles, each code times its
 *  scale converted exactly to bf16 in registers, which needs H and I of at
 *  least 128 and T*k*max(H, I)*2 below 2^31 (MOE_E_UNSUPPORTED otherwise).
 *  The global scale multiplies the fp32 sums of each row.
 *  For MOE_W_MXFP4 (the OCP microscaling sibling of NVFP4: the same E2M1
 *  codes with a power-of-two scale per 32 instead of an E4M3 one per 16) the
 *  codes are packed as for NVFP4, w_*_scales are E8M0 bytes [E, N, K/32],
 *  2^(b - 127) each (0xFF is NaN), one per 32 inputs, the weight is
 *  e2m1 * scale, exact in bf16 (for scale bytes below 253), and
 *  w_*_biases and the global scales are unused. Decode-sized batches
 *  stream the codes and scale each lane's 32-input partial in fp32; larger
 *  ones take the MFMA tiles as NVFP4 does, under the same conditions.
 *  shared_up   bf16 [2*I_shared, H] (SwiGLU, gate rows first) or
 *              [I_shared, H] (relu^2); shared_down bf16 [H, I_shared].
 *  w_up_tiles, w_down_tiles  optional (NULL: none), bf16 and block-FP8
 *              experts only: the tile-packed copies of w_up and w_down that
 *              moe_pack_tiles writes. Given, prompt-sized batches' MFMA
 *              tiles read their expert weights there (each K-slice of a
 *              tile is one contiguous 16 KB, 8 KB for FP8) and give the same
 *              bits as without them; w_up and w_down (and the FP8 scales)
 *              are still required and still read by the decode form, the
 *              shared expert and every other path. */
typedef struct {
    const float *router_w;
    const float *expert_bias;
    const void *w_up;
    const void *w_up_scales;       /* bf16 (MOE_W_AFFINE4) or fp32 (MOE_W_FP8) */
    const uint16_t *w_up_biases;
    const void *w_down;
    const void *w_down_scales;
    const uint16_t *w_down_biases;
    const uint16_t *shared_up;
    const uint16_t *shared_down;
    const float *w_up_global;      /* MOE_W_NVFP4: fp32 [E]; otherwise unused */
    const float *w_down_global;
    const void *w_up_tiles;        /* moe_pack_tiles(MOE_TILES_UP) of w_up, or NULL */
    const void *w_down_tiles;      /* moe_pack_tiles(MOE_TILES_DOWN) of w_down, or NULL */
} moe_weights;

/* Bytes of workspace moe_forward() and moe_plan() need for these dims. With
 * 4-bit experts and more than 2 E assignments (T * k > 2 E) or
 * row_invariant, and with block-FP8 experts whose max(H, I) exceeds 8192
 * (and, at decode sizes, 4096), this includes room for the bf16-decoded weights of every
 * expert that can have rows: min(E, T * k) * max(n_up * H, H * I) * 2 bytes,
 * n_up = 2 I (SwiGLU) or I. Otherwise the codes are read as stored. With a
 * shared expert whose I_shared is a whole number m of I, prompt-sized
 * batches also hold its m segments' rows: m*T more rows of h and y. */
int moe_workspace_bytes(const moe_dims *d, size_t *bytes);

/* Tile-packed expert weights (bf16 or block-FP8 codes), written once when
 * the weights are loaded, for the grouped GEMMs of the gate_up and down
 * projections (TileGym PR #187, "Weight layout and routing": w_up and w_down
 * as the caller stores them; the packed order is this library's). The MFMA
 * tiles take 256 weight rows at a time (SwiGLU: 128 gate rows, then the 128
 * up rows of the same columns) and 32 weights of each row per K-slice; in
 * the caller's layout those 16 KB (bf16) lie in 256 pieces of 64 bytes, 2K
 * bytes apart. The packed copy stores them in the order a stage holds them:
 *   bf16: tiles[e][nt][ks][s], 16 bytes per s = 0 .. 1023:
 *     row r = s / 4 of n-tile nt, chunk c = (s % 4) xor ((r / 4) % 4),
 *     that is weights 32 ks + 8 c .. + 7 of expert row
 *       SwiGLU up:  n = 128 nt + r % 128 (clamped to I - 1), row n for
 *                   r < 128, else row I + n
 *       otherwise:  256 nt + r, clamped to N - 1
 *   nt < ceil(I / 128) (SwiGLU up) or ceil(N / 256), ks < K / 32.
 *   FP8: the same with 16 codes per slot and two slots per row and slice,
 *     s = 0 .. 511: row r = s / 2, chunk c = (s % 2) xor ((r / 8) % 2),
 *     codes 32 ks + 16 c .. + 15.
 * which: MOE_TILES_UP packs w_up (N = 2I or I rows of H), MOE_TILES_DOWN
 * w_down (N = H rows of I). moe_tiles_bytes gives the size:
 * E * n_tiles * K * 512 bytes for bf16, half that for FP8 (rows past N are
 * stored as copies of the last row, so a ragged N costs up to 255 rows per
 * expert). moe_pack_tiles enqueues the copy on stream (w and tiles device
 * memory, 16-byte aligned, not overlapping). d is checked as for
 * moe_forward, and H, I, E, act and wfmt shape the copy; wfmt must be
 * MOE_W_BF16 or MOE_W_FP8 (MOE_E_UNSUPPORTED otherwise); MOE_E_WORKSPACE if
 * tiles_bytes is short. The copy is valid while w is unchanged. */
typedef enum { MOE_TILES_UP = 0, MOE_TILES_DOWN = 1 } moe_tiles_which;
int moe_tiles_bytes(const moe_dims *d, int32_t which, size_t *bytes);
int moe_pack_tiles(const moe_dims *d, int32_t which, const void *w, void *tiles,
                   size_t tiles_bytes, hipStream_t stream);

/* Router and top-k (TileGym PR #187 "Weight layout and routing"; TensorFold
 * PR #1492 "What").
 *  x        bf16 [T, H]
 *  ids      int32 [T, k]: the picks, best key first; equal keys go to the
 *           lower index; a NaN key ranks below every number, so an all-NaN
 *           row picks 0, 1, ..., k-1 (TensorFold PR #1492 "Verification")
 *  weights  fp32 [T, k]: unbiased scores, normalised when d->norm_topk;
 *           routed_scale is not applied here.
 * Workspace: moe_workspace_bytes(d) (the router uses T*E*4 bytes of it, or
 * T*E*(H/64)*4 when T <= 8 and E <= 32: the partial logits of every slice).
 * Only T, H, E, k, score_fn, norm_topk and norm_eps of d are read. A NaN
 * logit makes every softmax score of its row NaN (picks 0, 1, ..., k-1). */
int moe_route(const moe_dims *d, const uint16_t *x, const float *router_w,
              const float *expert_bias, int32_t *ids, float *weights, void *workspace,
              size_t workspace_bytes, hipStream_t stream);

/* Expert plan (TensorFold issue #548, the grouped expert plan): histogram,
 * exclusive scan and a stable permutation of the assignments a = t*k + j
 * into per-expert segments.
 *  ids      int32 [T, k]
 *  counts   int32 [E]
 *  offsets  int32 [E+1], offsets[E] = number of in-range assignments
 *  sorted   int32 [T*k]: assignment indices, expert-major, ascending a inside
 *           an expert; entries past offsets[E] are set to -1
 *  slot_of  int32 [T*k]: the position of each assignment in sorted, or -1
 *  fault    int32 [1] or NULL: incremented by the number of ids outside
 *           [0, E); such assignments are left out of every segment (the
 *           caller reads it back after the stream completes)
 * Workspace: moe_workspace_bytes(d). */
int moe_plan(const moe_dims *d, const int32_t *ids, int32_t *counts, int32_t *offsets,
             int32_t *sorted, int32_t *slot_of, int32_t *fault, void *workspace,
             size_t workspace_bytes, hipStream_t stream);

/* The whole block: route, plan, grouped expert GEMMs with the activation
 * fused into the first, the shared expert, and the weighted combine.
 *  x    bf16 [T, H]
 *  out  [T, H], bf16 or fp32 by d->out_dtype: each element is computed in
 *       fp32 as routed_scale * (fma chain of w_j * y_j, j ascending), plus
 *       the shared expert's output, and rounded once; with
 *       d->fold_routed_scale, as the fma chain of (routed_scale * w_j) * y_j,
 *       j ascending. weights_out holds the unscaled w_j either way. When
 *       I_shared is a whole number m of I, prompt-sized batches run the
 *       shared expert as m segments of every token inside the routed
 *       experts' launches (the plan's extra slots), and its output is the
 *       sum of the m partial rows, v ascending.
 *  ids_out, weights_out ([T, k]) and offsets_out ([E+1]) may be NULL; when
 *  given they receive the routing and the plan offsets of this call.
 * Workspace: moe_workspace_bytes(d). */
int moe_forward(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                void *workspace, size_t workspace_bytes, hipStream_t stream,
                int32_t *ids_out, float *weights_out, int32_t *offsets_out);

/* moe_forward, with stage boundaries recorded on the stream for timing:
 * events[0] before the router, [1] after the router, [2] after the plan,
 * [3] after the routed up-projection GEMM (gate_up + SwiGLU, or up +
 * relu^2), [4] after the routed down GEMM, [5] after the shared expert
 * (same as [4] without one), [6] after the combine. Each entry is a
 * hipEvent_t created by the caller, or NULL to skip it. The bf16 decode form
 * (T*k <= 32, I <= 2048) runs the shared expert before the routed up
 * projection and the combine inside the down GEMM's launch: there [4], [5]
 * and [6] follow that launch back to back. */
#define MOE_PROFILE_EVENTS 7
int moe_forward_profiled(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         int32_t *ids_out, float *weights_out, int32_t *offsets_out,
                         hipEvent_t events[MOE_PROFILE_EVENTS]);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same block and the same kernels, with the workspace taken
 * from a static device array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends. The entry point
 * calls no allocator. Inputs and outputs are as for moe_forward; the
 * current device must be the one the stream and the tensors belong to.
 * Calls whose workspace (moe_workspace_bytes) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES are refused with MOE_E_WORKSPACE before
 * anything is enqueued (4-bit experts of prompt-sized batches and block-FP8
 * experts need room for decoded weights and usually are). Every call on one
 * GPU shares that GPU's scratch: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be
 * issued. A call does not rely on anything a previous call left there. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                        hipStream_t stream, int32_t *ids_out, float *weights_out,
                        int32_t *offsets_out);

/* Fused residual add + RMSNorm, the step that makes the block's input x
 * (TensorFold issue #548: RMSNorm and the fused add + RMSNorm among the shared
 * layer pieces, a row's bits the same at every row count; TensorFold PR #1492:
 * the reused addRmsTail norms). For each of the T rows of H:
 *   r            = h + residual        fp32 sum of the bf16 values (r = residual if h is NULL)
 *   residual_out = bf16(r)             round to nearest even: the residual stream
 *   x            = bf16(r * gamma / sqrt(sum(r^2) / H + eps))
 *  h, residual, residual_out, x  bf16 [T, H]; gamma bf16 [H]
 *  h and residual_out may be NULL (then plain RMSNorm, residual not rewritten);
 *  residual_out may equal residual (in place); no other two may overlap.
 *  Limits: 0 <= T <= 2^24; H a multiple of 64, at most 8192; eps finite, >= 0.
 * A row's outputs depend on that row only (one wavefront per row), so they
 * are the same bits at any T. Same error and stream conventions as above; no
 * workspace. */
int moe_add_rmsnorm(int32_t T, int32_t H, const uint16_t *h, const uint16_t *residual,
                    const uint16_t *gamma, float eps, uint16_t *residual_out, uint16_t *x,
                    hipStream_t stream);

/* Text of the last error on this thread ("" after a success). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
