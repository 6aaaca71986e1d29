// api.cpp -- the C ABI declared in include/moe.h: argument checks, the
// workspace layout and the order of launches.
//
// The checks follow the refusal style of the pages' hosts: every size and
// pointer is checked before anything is enqueued, and the error text names
// the argument, what it got and what it needed (bloomery PR #235, review of
// enqueue_pass; vllm.cpp PR #684: a tensor that is not device memory is
// refused on the host, outputs are f32 or bf16 only).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int ok() {
    g_error.clear();
    return MOE_OK;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t z, ids, w, counts, offsets, seg_offsets, sorted, slot, chunk_counts, h, y, hs, ys, wdq,
        total;
};

// Decode-sized batches (at most two assignments per expert on average)
// stream each touched expert's weights once; larger ones take the MFMA tiles
// (TensorFold issue #548: decode rows and prompt rows).
// With row_invariant no batch is: every one takes the tiles.
bool decode_sized(const moe_dims &d) {
    return !d.row_invariant && (int64_t)d.T * d.k <= 2 * (int64_t)d.E;
}

// Quantized experts the decode form streams at their stored width (the
// projections' K within its limits).
bool quant_streams(const moe_dims &d) {
    const int kmax = std::max(d.H, d.I);
    return decode_sized(d) && ((d.wfmt == MOE_W_AFFINE4 && kmax <= moe::kStreamMaxKAffine4) ||
                               (d.wfmt == MOE_W_FP8 && kmax <= moe::kStreamMaxKFp8) ||
                               (d.wfmt == MOE_W_NVFP4 && kmax <= moe::kStreamMaxKNvfp4) ||
                               (d.wfmt == MOE_W_MXFP4 && kmax <= moe::kStreamMaxKMxfp4));
}

// Block-FP8 experts the persistent MFMA kernel reads at their stored width
// (one byte per weight, the block scales applied to the fp32 sums): the
// scales of a row block's K-blocks fit one per lane (K <= 64 x 128).
bool fp8_tiles(const moe_dims &d) {
    return d.wfmt == MOE_W_FP8 && d.H <= 64 * 128 && d.I <= 64 * 128;
}

// NVFP4 and MXFP4 experts the persistent MFMA kernel reads at their stored
// width (half a byte per weight, each code times its scale converted
// exactly to bf16 in registers): every batch the decode form does not take,
// within the kernel's 32-bit row offsets.
bool f4_tiles(const moe_dims &d) {
    return (d.wfmt == MOE_W_NVFP4 || d.wfmt == MOE_W_MXFP4) && !quant_streams(d) &&
           d.H >= 128 && d.I >= 128 &&
           (int64_t)d.T * d.k * std::max(d.H, d.I) * 2 < ((int64_t)1 << 31);
}

// 4-bit experts of prompt-sized batches, and block-FP8 experts that neither
// the decode form nor the FP8 tiles take, are decoded to bf16 (the weights
// of the experts with rows, once per call) before the bf16 MFMA kernel
// runs. Decode-sized 4-bit batches the stream does not take keep the decode
// in the staged kernel's loads. (NVFP4 and MXFP4 batches take the stream or
// their tiles; check_dims refuses the shapes neither takes.)
bool dequant_first(const moe_dims &d) {
    return (d.wfmt == MOE_W_AFFINE4 && !decode_sized(d)) ||
           (d.wfmt == MOE_W_FP8 && !quant_streams(d) && !fp8_tiles(d));
}

// The shared expert as m plan segments of the routed experts' width
// (I_shared = m I), run inside the routed experts' grouped launches: every
// token is a row of each segment, segment v taking gate/up rows v I .. and
// down columns v I .. of the shared weights (vllm.cpp PR #684, the 9-slot
// plan of the top-k plus the shared id). Prompt-sized batches on the MFMA
// tiles with bf16 or decoded 4-bit experts; 0 otherwise (the shared expert
// then runs as its own dense projections).
int shared_segments(const moe_dims &d) {
    if (d.I_shared <= 0 || d.I_shared % d.I != 0 || decode_sized(d) || d.wfmt == MOE_W_FP8 ||
        f4_tiles(d))
        return 0;
    const int m = d.I_shared / d.I;
    const int64_t rows = (int64_t)d.T * d.k + (int64_t)m * d.T;   // plan positions
    const int64_t up_rows = (rows + d.k - 1) / d.k;                // bound of the gathered rows
    if (d.E + m > 256 || d.H < 128 || d.I < 128 || up_rows * d.H * 2 >= ((int64_t)1 << 31) ||
        rows * d.I * 2 >= ((int64_t)1 << 31))
        return 0;
    return m;
}

Layout layout(const moe_dims &d) {
    Layout L{};
    const size_t A = (size_t)d.T * d.k;
    const int m = shared_segments(d);
    const size_t R = A + (size_t)m * d.T;      // plan positions, shared segments included
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += round_up(bytes);
        return o;
    };
    L.z = take(moe::route_scratch_bytes(d.T, d.H, d.E));
    L.ids = take(A * 4);
    L.w = take(A * 4);
    L.counts = take((size_t)d.E * 4);
    L.offsets = take((size_t)(d.E + 1) * 4);
    if (m > 0)
        L.seg_offsets = take((size_t)(d.E + m + 1) * 4);
    L.sorted = take(R * 4);
    L.slot = take(A * 4);
    L.chunk_counts = take((size_t)moe::plan_chunks((int)A) * d.E * 4);
    L.h = take(((R + 15) & ~(size_t)15) * d.I * 2);   // whole row blocks of 16
    L.y = take(R * d.H * 4);
    if (d.I_shared > 0 && m == 0) {
        L.hs = take((size_t)d.T * d.I_shared * 2);
        L.ys = take((size_t)d.T * d.H * 4);
    }
    if (dequant_first(d)) {
        // the bf16 weights of the experts with rows, one projection at a time
        const size_t experts = (size_t)(A < (size_t)d.E ? A : d.E);
        const size_t n_up = d.act == MOE_ACT_SWIGLU ? 2 * (size_t)d.I : (size_t)d.I;
        const size_t per = n_up * d.H > (size_t)d.H * d.I ? n_up * d.H : (size_t)d.H * d.I;
        L.wdq = take(experts * per * 2);
    }
    L.total = off;
    return L;
}

bool aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...)              \
    do {                                      \
        if (!(cond))                          \
            return fail((code), __VA_ARGS__); \
    } while (0)

// Shape checks shared by every entry point. `what` names the caller.
int check_dims(const char *what, const moe_dims *d, bool experts) {
    REQUIRE(d != nullptr, MOE_E_NULL, "%s: dims is NULL", what);
    REQUIRE(d->T >= 0 && d->T <= (1 << 24), MOE_E_SHAPE, "%s: T = %d, need 0 <= T <= 2^24", what,
            d->T);
    REQUIRE(d->H > 0 && d->H % 64 == 0 && d->H <= 65536, MOE_E_SHAPE,
            "%s: H = %d, need a positive multiple of 64 up to 65536", what, d->H);
    REQUIRE(d->E >= 1 && d->E <= 256, MOE_E_SHAPE, "%s: E = %d, need 1 <= E <= 256", what, d->E);
    REQUIRE(d->k >= 1 && d->k <= 8 && d->k <= d->E, MOE_E_SHAPE,
            "%s: k = %d, need 1 <= k <= min(E = %d, 8)", what, d->k, d->E);
    REQUIRE((int64_t)d->T * d->k * d->H < ((int64_t)1 << 31), MOE_E_SHAPE,
            "%s: T*k*H = %lld, need < 2^31", what, (long long)d->T * d->k * d->H);
    REQUIRE(d->norm_topk == 0 || d->norm_topk == 1, MOE_E_UNSUPPORTED,
            "%s: norm_topk = %d, need 0 or 1", what, d->norm_topk);
    REQUIRE(std::isfinite(d->norm_eps) && d->norm_eps >= 0.0f, MOE_E_SHAPE,
            "%s: norm_eps = %g, need a finite value >= 0", what, (double)d->norm_eps);
    REQUIRE(d->score_fn == MOE_SCORE_SIGMOID || d->score_fn == MOE_SCORE_SOFTMAX,
            MOE_E_UNSUPPORTED, "%s: score_fn = %d, need MOE_SCORE_SIGMOID (0) or "
            "MOE_SCORE_SOFTMAX (1)", what, d->score_fn);
    if (!experts)
        return MOE_OK;
    REQUIRE(d->I > 0 && d->I % 64 == 0 && d->I <= 65536, MOE_E_SHAPE,
            "%s: I = %d, need a positive multiple of 64 up to 65536", what, d->I);
    REQUIRE(d->I_shared >= 0 && d->I_shared % 64 == 0 && d->I_shared <= 65536, MOE_E_SHAPE,
            "%s: I_shared = %d, need 0 or a positive multiple of 64 up to 65536", what,
            d->I_shared);
    REQUIRE((int64_t)d->T * d->k * d->I < ((int64_t)1 << 31) &&
                (int64_t)d->T * d->I_shared < ((int64_t)1 << 31),
            MOE_E_SHAPE, "%s: T*k*I or T*I_shared reaches 2^31", what);
    REQUIRE((int64_t)2 * std::max(d->I, d->I_shared) * d->H < ((int64_t)1 << 31), MOE_E_SHAPE,
            "%s: 2*max(I, I_shared)*H reaches 2^31 (one expert's weight matrix)", what);
    REQUIRE(d->act == MOE_ACT_SWIGLU || d->act == MOE_ACT_RELU2, MOE_E_UNSUPPORTED,
            "%s: act = %d, need MOE_ACT_SWIGLU (0) or MOE_ACT_RELU2 (1)", what, d->act);
    REQUIRE(d->wfmt == MOE_W_BF16 || d->wfmt == MOE_W_AFFINE4 || d->wfmt == MOE_W_FP8 ||
                d->wfmt == MOE_W_NVFP4 || d->wfmt == MOE_W_MXFP4,
            MOE_E_UNSUPPORTED, "%s: wfmt = %d, need MOE_W_BF16 (0), MOE_W_AFFINE4 (1), "
            "MOE_W_FP8 (2), MOE_W_NVFP4 (3) or MOE_W_MXFP4 (4)", what, d->wfmt);
    if (d->wfmt == MOE_W_FP8) {
        REQUIRE(d->H % 128 == 0 && d->I % 128 == 0, MOE_E_SHAPE,
                "%s: H = %d, I = %d: block-FP8 experts need multiples of 128", what, d->H, d->I);
        // the decoded weights run on the MFMA kernel, whose row offsets are 32-bit bytes
        REQUIRE((int64_t)d->T * d->k * std::max(d->H, d->I) * 2 < ((int64_t)1 << 31),
                MOE_E_SHAPE, "%s: T*k*max(H, I)*2 reaches 2^31 with block-FP8 experts", what);
    }
    if (d->wfmt == MOE_W_AFFINE4)
        REQUIRE(d->group == 64, MOE_E_UNSUPPORTED, "%s: group = %d, the 4-bit format needs 64",
                what, d->group);
    if (d->wfmt == MOE_W_NVFP4 || d->wfmt == MOE_W_MXFP4)
        REQUIRE(quant_streams(*d) || f4_tiles(*d), MOE_E_UNSUPPORTED,
                "%s: NVFP4 / MXFP4 experts: a batch the weight-streaming form does not take "
                "(T*k = %lld > 2E, row_invariant, or H or I past 8192) needs H, I >= 128 and "
                "T*k*max(H, I)*2 < 2^31 for the MFMA tiles (H = %d, I = %d)",
                what, (long long)d->T * d->k, d->H, d->I);
    REQUIRE(d->out_dtype == MOE_OUT_BF16 || d->out_dtype == MOE_OUT_F32, MOE_E_UNSUPPORTED,
            "%s: out_dtype = %d, need MOE_OUT_BF16 (0) or MOE_OUT_F32 (1)", what, d->out_dtype);
    REQUIRE(std::isfinite(d->routed_scale), MOE_E_SHAPE, "%s: routed_scale = %g is not finite",
            what, (double)d->routed_scale);
    REQUIRE(std::isfinite(d->swiglu_limit) && d->swiglu_limit >= 0.0f, MOE_E_SHAPE,
            "%s: swiglu_limit = %g, need a finite value >= 0", what, (double)d->swiglu_limit);
    REQUIRE(d->swiglu_limit == 0.0f || d->act == MOE_ACT_SWIGLU, MOE_E_UNSUPPORTED,
            "%s: swiglu_limit = %g applies to MOE_ACT_SWIGLU only (act = %d)", what,
            (double)d->swiglu_limit, d->act);
    REQUIRE(d->fold_routed_scale == 0 || d->fold_routed_scale == 1, MOE_E_UNSUPPORTED,
            "%s: fold_routed_scale = %d, need 0 or 1", what, d->fold_routed_scale);
    REQUIRE(d->row_invariant == 0 || d->row_invariant == 1, MOE_E_UNSUPPORTED,
            "%s: row_invariant = %d, need 0 or 1", what, d->row_invariant);
    REQUIRE(d->fold_routed_scale == 0 || d->I_shared == 0, MOE_E_UNSUPPORTED,
            "%s: fold_routed_scale = 1 with I_shared = %d: the fold is legal only without "
            "a shared expert", what, d->I_shared);
    return MOE_OK;
}

// A required device tensor: not NULL, 16-byte aligned.
int check_ptr(const char *what, const char *name, const void *p) {
    REQUIRE(p != nullptr, MOE_E_NULL, "%s: %s is NULL", what, name);
    REQUIRE(aligned(p), MOE_E_ALIGN, "%s: %s = %p is not 16-byte aligned", what, name, p);
    return MOE_OK;
}

int check_opt_ptr(const char *what, const char *name, const void *p) {
    REQUIRE(p == nullptr || aligned(p), MOE_E_ALIGN, "%s: %s = %p is not 16-byte aligned", what,
            name, p);
    return MOE_OK;
}

// Device allocations this thread has validated: a pointer inside one is not
// queried again. A call makes up to 16 pointer checks, which cost more host
// time than the launches of a decode step; the weights, workspace and
// outputs of a layer repeat from call to call, so after the first call none
// is queried. (A pointer into memory freed since is not caught; that is
// undefined anyway.)
struct DevRange {
    uintptr_t lo, hi;
};
constexpr int kDevRanges = 64;
thread_local DevRange t_dev_ranges[kDevRanges];
thread_local int t_dev_count = 0;
thread_local int t_dev_next = 0;

bool known_device(const void *p) {
    const uintptr_t a = (uintptr_t)p;
    for (int i = 0; i < t_dev_count; ++i)
        if (a >= t_dev_ranges[i].lo && a < t_dev_ranges[i].hi)
            return true;
    return false;
}

void remember_device(const void *p) {
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess || size == 0) {
        (void)hipGetLastError();
        return;
    }
    t_dev_ranges[t_dev_next] = DevRange{(uintptr_t)base, (uintptr_t)base + size};
    t_dev_next = (t_dev_next + 1) % kDevRanges;
    if (t_dev_count < kDevRanges)
        ++t_dev_count;
}

// Device memory check, the last check before launching (it is the only one
// that asks the HIP runtime).
int check_device(const char *what, const char *name, const void *p) {
    if (p == nullptr || known_device(p))
        return MOE_OK;
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_E_SHAPE, "%s: %s = %p is not memory the HIP runtime knows (%s)", what,
                    name, p, hipGetErrorString(e));
    }
    REQUIRE(attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged, MOE_E_SHAPE,
            "%s: %s = %p is not device memory", what, name, p);
    remember_device(p);
    return MOE_OK;
}

#define TRY(expr)                 \
    do {                          \
        const int rc_ = (expr);   \
        if (rc_ != MOE_OK)        \
            return rc_;           \
    } while (0)

#define LAUNCH(expr)                                                                       \
    do {                                                                                   \
        const hipError_t e_ = (expr);                                                      \
        if (e_ != hipSuccess)                                                              \
            return fail(MOE_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e_)); \
    } while (0)

// The tensor moe_pack_tiles packs: rows N, row length K and whether it is a
// fused gate/up tensor.
struct PackShape {
    int N, K, I;
    bool gate_up;
    int esz;                       // bytes per weight: 2 (bf16) or 1 (FP8 codes)
};
int pack_shape(const char *what, const moe_dims *d, int32_t which, PackShape *ps) {
    TRY(check_dims(what, d, true));
    REQUIRE(d->wfmt == MOE_W_BF16 || d->wfmt == MOE_W_FP8, MOE_E_UNSUPPORTED,
            "%s: wfmt = %d, the tile-packed copy is for bf16 and block-FP8 experts", what,
            d->wfmt);
    REQUIRE(which == MOE_TILES_UP || which == MOE_TILES_DOWN, MOE_E_UNSUPPORTED,
            "%s: which = %d, need MOE_TILES_UP (0) or MOE_TILES_DOWN (1)", what, which);
    const bool swiglu = d->act == MOE_ACT_SWIGLU;
    const int esz = d->wfmt == MOE_W_FP8 ? 1 : 2;
    if (which == MOE_TILES_UP)
        *ps = PackShape{swiglu ? 2 * d->I : d->I, d->H, d->I, swiglu, esz};
    else
        *ps = PackShape{d->H, d->I, d->I, false, esz};
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_workspace_bytes(const moe_dims *d, size_t *bytes) {
    const char *what = "moe_workspace_bytes";
    TRY(check_dims(what, d, true));
    REQUIRE(bytes != nullptr, MOE_E_NULL, "%s: bytes is NULL", what);
    *bytes = layout(*d).total;
    return ok();
}

int moe_tiles_bytes(const moe_dims *d, int32_t which, size_t *bytes) {
    const char *what = "moe_tiles_bytes";
    PackShape ps{};
    TRY(pack_shape(what, d, which, &ps));
    REQUIRE(bytes != nullptr, MOE_E_NULL, "%s: bytes is NULL", what);
    *bytes = moe::pack_tiles_bytes(d->E, ps.N, ps.K, ps.I, ps.gate_up, ps.esz);
    return ok();
}

int moe_pack_tiles(const moe_dims *d, int32_t which, const void *w, void *tiles,
                   size_t tiles_bytes, hipStream_t stream) {
    const char *what = "moe_pack_tiles";
    PackShape ps{};
    TRY(pack_shape(what, d, which, &ps));
    const size_t need = moe::pack_tiles_bytes(d->E, ps.N, ps.K, ps.I, ps.gate_up, ps.esz);
    REQUIRE(tiles_bytes >= need, MOE_E_WORKSPACE, "%s: tiles_bytes = %zu, need >= %zu", what,
            tiles_bytes, need);
    TRY(check_ptr(what, "w", w));
    TRY(check_ptr(what, "tiles", tiles));
    TRY(check_device(what, "w", w));
    TRY(check_device(what, "tiles", tiles));
    LAUNCH(moe::launch_pack_tiles(w, tiles, d->E, ps.N, ps.K, ps.I, ps.gate_up, ps.esz, stream));
    return ok();
}

int moe_route(const moe_dims *d, const uint16_t *x, const float *router_w,
              const float *expert_bias, int32_t *ids, float *weights, void *workspace,
              size_t workspace_bytes, hipStream_t stream) {
    const char *what = "moe_route";
    TRY(check_dims(what, d, false));
    if (d->T == 0)
        return ok();
    TRY(check_ptr(what, "x", x));
    TRY(check_ptr(what, "router_w", router_w));
    TRY(check_opt_ptr(what, "expert_bias", expert_bias));
    TRY(check_ptr(what, "ids", ids));
    TRY(check_ptr(what, "weights", weights));
    // the router needs only the logits scratch of the layout
    const size_t need = round_up(moe::route_scratch_bytes(d->T, d->H, d->E));
    REQUIRE(workspace_bytes >= need, MOE_E_WORKSPACE, "%s: workspace_bytes = %zu, need >= %zu",
            what, workspace_bytes, need);
    TRY(check_ptr(what, "workspace", workspace));
    for (const auto &pr : {std::make_pair("x", (const void *)x),
                           std::make_pair("router_w", (const void *)router_w),
                           std::make_pair("expert_bias", (const void *)expert_bias),
                           std::make_pair("ids", (const void *)ids),
                           std::make_pair("weights", (const void *)weights),
                           std::make_pair("workspace", (const void *)workspace)})
        TRY(check_device(what, pr.first, pr.second));
    LAUNCH(moe::launch_route(x, router_w, expert_bias, d->T, d->H, d->E, d->k, d->score_fn,
                             d->norm_topk, d->norm_eps, ids, weights, (float *)workspace,
                             moe::PlanOut{}, nullptr, stream));
    return ok();
}

int moe_plan(const moe_dims *d, const int32_t *ids, int32_t *counts, int32_t *offsets,
             int32_t *sorted, int32_t *slot_of, int32_t *fault, void *workspace,
             size_t workspace_bytes, hipStream_t stream) {
    const char *what = "moe_plan";
    TRY(check_dims(what, d, false));
    const int A = d->T * d->k;
    TRY(check_ptr(what, "counts", counts));
    TRY(check_ptr(what, "offsets", offsets));
    TRY(check_opt_ptr(what, "fault", fault));
    if (A > 0) {
        TRY(check_ptr(what, "ids", ids));
        TRY(check_ptr(what, "sorted", sorted));
        TRY(check_ptr(what, "slot_of", slot_of));
    }
    // the plan needs only the per-chunk counts of the layout
    const size_t need = round_up((size_t)moe::plan_chunks(A) * d->E * 4);
    REQUIRE(workspace_bytes >= need, MOE_E_WORKSPACE, "%s: workspace_bytes = %zu, need >= %zu",
            what, workspace_bytes, need);
    if (need > 0)
        TRY(check_ptr(what, "workspace", workspace));
    for (const auto &pr : {std::make_pair("ids", (const void *)ids),
                           std::make_pair("counts", (const void *)counts),
                           std::make_pair("offsets", (const void *)offsets),
                           std::make_pair("sorted", (const void *)sorted),
                           std::make_pair("slot_of", (const void *)slot_of),
                           std::make_pair("fault", (const void *)fault),
                           std::make_pair("workspace", (const void *)workspace)})
        TRY(check_device(what, pr.first, pr.second));
    LAUNCH(moe::launch_plan(ids, A, d->E, counts, offsets, sorted, slot_of, fault,
                            (int32_t *)workspace, stream));
    return ok();
}

namespace {

int forward_impl(const char *what, const moe_dims *d, const moe_weights *w, const uint16_t *x,
                 void *out, void *workspace, size_t workspace_bytes, hipStream_t stream,
                 int32_t *ids_out, float *weights_out, int32_t *offsets_out, hipEvent_t *events,
                 bool workspace_is_scratch = false) {
    TRY(check_dims(what, d, true));
    REQUIRE(w != nullptr, MOE_E_NULL, "%s: weights is NULL", what);
    TRY(check_ptr(what, "w->router_w", w->router_w));
    TRY(check_opt_ptr(what, "w->expert_bias", w->expert_bias));
    TRY(check_ptr(what, "w->w_up", w->w_up));
    TRY(check_ptr(what, "w->w_down", w->w_down));
    const bool aff = d->wfmt == MOE_W_AFFINE4;
    const bool fp8 = d->wfmt == MOE_W_FP8;
    const bool nv4 = d->wfmt == MOE_W_NVFP4;
    const bool mx4 = d->wfmt == MOE_W_MXFP4;
    if (fp8 || nv4 || mx4) {
        TRY(check_ptr(what, "w->w_up_scales", w->w_up_scales));
        TRY(check_ptr(what, "w->w_down_scales", w->w_down_scales));
    }
    if (nv4) {
        REQUIRE(w->w_up_global != nullptr && w->w_down_global != nullptr, MOE_E_NULL,
                "%s: NVFP4 experts need w->w_up_global and w->w_down_global", what);
    }
    if (aff) {
        TRY(check_ptr(what, "w->w_up_scales", w->w_up_scales));
        TRY(check_ptr(what, "w->w_up_biases", w->w_up_biases));
        TRY(check_ptr(what, "w->w_down_scales", w->w_down_scales));
        TRY(check_ptr(what, "w->w_down_biases", w->w_down_biases));
    }
    if (d->I_shared > 0) {
        TRY(check_ptr(what, "w->shared_up", w->shared_up));
        TRY(check_ptr(what, "w->shared_down", w->shared_down));
    }
    REQUIRE((w->w_up_tiles == nullptr && w->w_down_tiles == nullptr) || d->wfmt == MOE_W_BF16 ||
                d->wfmt == MOE_W_FP8,
            MOE_E_UNSUPPORTED,
            "%s: w->w_up_tiles / w->w_down_tiles are for bf16 and block-FP8 experts (wfmt = %d)",
            what, d->wfmt);
    TRY(check_opt_ptr(what, "w->w_up_tiles", w->w_up_tiles));
    TRY(check_opt_ptr(what, "w->w_down_tiles", w->w_down_tiles));
    TRY(check_opt_ptr(what, "ids_out", ids_out));
    TRY(check_opt_ptr(what, "weights_out", weights_out));
    TRY(check_opt_ptr(what, "offsets_out", offsets_out));
    const Layout L = layout(*d);
    REQUIRE(workspace_bytes >= L.total, MOE_E_WORKSPACE, "%s: workspace_bytes = %zu, need >= %zu",
            what, workspace_bytes, L.total);
    if (d->T == 0)
        return ok();
    TRY(check_ptr(what, "x", x));
    TRY(check_ptr(what, "out", out));
    TRY(check_ptr(what, "workspace", workspace));
    // (the static scratch is a device global, not an allocation the
    // runtime's pointer query knows)
    const void *dev[] = {x, out, workspace_is_scratch ? nullptr : workspace, w->router_w, w->expert_bias, w->w_up, w->w_down,
                         aff || fp8 || nv4 || mx4 ? w->w_up_scales : nullptr,
                         aff ? w->w_up_biases : nullptr,
                         aff || fp8 || nv4 || mx4 ? w->w_down_scales : nullptr,
                         aff ? w->w_down_biases : nullptr,
                         d->I_shared ? w->shared_up : nullptr,
                         d->I_shared ? w->shared_down : nullptr, ids_out, weights_out,
                         offsets_out, nv4 ? w->w_up_global : nullptr,
                         nv4 ? w->w_down_global : nullptr, w->w_up_tiles, w->w_down_tiles};
    const char *dev_names[] = {"x", "out", "workspace", "w->router_w", "w->expert_bias",
                               "w->w_up", "w->w_down", "w->w_up_scales", "w->w_up_biases",
                               "w->w_down_scales", "w->w_down_biases", "w->shared_up",
                               "w->shared_down", "ids_out", "weights_out", "offsets_out",
                               "w->w_up_global", "w->w_down_global", "w->w_up_tiles",
                               "w->w_down_tiles"};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
        TRY(check_device(what, dev_names[i], dev[i]));

    char *ws = (char *)workspace;
    const int T = d->T, H = d->H, I = d->I, E = d->E, k = d->k, A = T * k;
    int32_t *ids = ids_out ? ids_out : (int32_t *)(ws + L.ids);
    float *wts = weights_out ? weights_out : (float *)(ws + L.w);
    int32_t *counts = (int32_t *)(ws + L.counts);
    int32_t *offsets = offsets_out ? offsets_out : (int32_t *)(ws + L.offsets);
    int32_t *sorted = (int32_t *)(ws + L.sorted);
    int32_t *slot = (int32_t *)(ws + L.slot);
    uint16_t *h = (uint16_t *)(ws + L.h);
    float *y = (float *)(ws + L.y);
    const int m = shared_segments(*d);
    int32_t *seg_off = m > 0 ? (int32_t *)(ws + L.seg_offsets) : offsets;
    const int R = A + m * T;                 // plan positions, shared segments included

    auto mark = [&](int i) -> hipError_t {
        return (events != nullptr && events[i] != nullptr) ? hipEventRecord(events[i], stream)
                                                           : hipSuccess;
    };
    LAUNCH(mark(0));
    bool plan_done = false;
    // (the router builds the plan itself only without shared segments)
    LAUNCH(moe::launch_route(x, w->router_w, w->expert_bias, T, H, E, k, d->score_fn,
                             d->norm_topk, d->norm_eps, ids, wts, (float *)(ws + L.z),
                             m > 0 ? moe::PlanOut{} : moe::PlanOut{counts, offsets, sorted, slot},
                             &plan_done, stream));
    LAUNCH(mark(1));
    if (!plan_done)
        LAUNCH(moe::launch_plan(ids, A, E, counts, offsets, sorted, slot, nullptr,
                                (int32_t *)(ws + L.chunk_counts), stream,
                                m > 0 ? seg_off : nullptr, m, T));
    LAUNCH(mark(2));
    const bool decode_form = decode_sized(*d);
    auto run = [&](const moe::GemmProblem &g) {
        return decode_form && moe::stream_supported(g) ? moe::launch_stream(g, stream)
                                                       : moe::launch_gemm(g, stream);
    };

    moe::GemmProblem up{};
    const int gate_mode = d->swiglu_limit > 0.0f ? moe::kGateUpLimit : moe::kGateUp;
    up.mode = d->act == MOE_ACT_SWIGLU ? gate_mode : moe::kUpRelu2;
    up.affine4 = aff;
    up.fp8 = d->wfmt == MOE_W_FP8;
    up.nvfp4 = nv4;
    up.mxfp4 = mx4;
    up.Bglobal = nv4 ? w->w_up_global : nullptr;
    up.A = x;
    up.lda = H;
    up.gather = sorted;
    up.gather_div = k;
    up.offsets = seg_off;
    up.E = E;
    up.max_rows = R;
    if (m > 0) {
        // segment E + v: gate rows v I .. (up rows I_shared + v I ..) of the
        // shared up projection
        up.B2 = (const uint16_t *)w->shared_up;
        up.E2 = m;
        up.b2_ld = H;
        up.b2_up = d->I_shared;
        up.b2_vstride = (long long)I * H;
    }
    up.B = w->w_up;
    up.Btiles = w->w_up_tiles;
    up.Bscale = (const uint16_t *)w->w_up_scales;
    up.Bbias = (const uint16_t *)w->w_up_biases;
    up.N = d->act == MOE_ACT_SWIGLU ? 2 * I : I;
    up.K = H;
    up.I = I;
    up.C = h;
    up.ldc = I;
    up.limit = d->swiglu_limit;
    // 4-bit weights, prompt-sized batch (dequant_first): decoded to bf16
    // first, then the bf16 kernel on the experts with rows
    uint16_t *wdq = (uint16_t *)(ws + L.wdq);
    auto dequantized = [&](moe::GemmProblem g) {
        g.affine4 = 0;
        g.fp8 = 0;
        g.nvfp4 = 0;                 // (an NVFP4 global scale stays in Bglobal)
        g.mxfp4 = 0;
        g.B = wdq;
        g.Btiles = nullptr;
        g.Bscale = nullptr;
        g.Bbias = nullptr;
        g.b_compact = 1;
        return g;
    };
    const bool dq = dequant_first(*d) && moe::grouped_supported(dequantized(up));

    moe::GemmProblem down{};
    down.mode = moe::kDown;
    down.affine4 = aff;
    down.fp8 = up.fp8;
    down.nvfp4 = nv4;
    down.mxfp4 = mx4;
    down.Bglobal = nv4 ? w->w_down_global : nullptr;
    down.A = h;
    down.lda = I;
    down.offsets = seg_off;
    down.E = E;
    down.max_rows = R;
    if (m > 0) {
        // segment E + v: columns v I .. v I + I - 1 of the shared down projection
        down.B2 = (const uint16_t *)w->shared_down;
        down.E2 = m;
        down.b2_ld = d->I_shared;
        down.b2_vstride = I;
    }
    down.B = w->w_down;
    down.Btiles = w->w_down_tiles;
    down.Bscale = (const uint16_t *)w->w_down_scales;
    down.Bbias = (const uint16_t *)w->w_down_biases;
    down.N = H;
    down.K = I;
    down.I = I;
    down.C = y;                        // rows in segment order: the combine gathers them
    down.ldc = H;

    // The bf16 decode form runs the down projection and the combine in one
    // launch (launch_down_combine); the shared expert, which reads only x,
    // then runs first.
    const bool fused = decode_form && !dq && moe::stream_supported(up) &&
                       moe::down_combine_supported(down, T, k);
    // h in row blocks of 16 (each K-slice of a block 1 KB in one piece) when
    // the persistent kernel both writes it (up) and reads it back (down)
    {
        const moe::GemmProblem up_run = dq ? dequantized(up) : up;
        const moe::GemmProblem down_run =
            dq && moe::grouped_supported(dequantized(down)) ? dequantized(down) : down;
        const bool up_tiles = !(decode_form && moe::stream_supported(up_run)) &&
                              moe::grouped_supported(up_run);
        const bool down_tiles = !fused && !(decode_form && moe::stream_supported(down_run)) &&
                                moe::grouped_supported(down_run);
        const bool blocked = up_tiles && down_tiles && I % 32 == 0 &&
                             ((int64_t)R + 16) * I * 2 < ((int64_t)1 << 31);
        up.c_blocked = blocked;
        down.a_blocked = blocked;
    }
    const float *shared = nullptr;
    int shared_terms = 1;
    auto run_shared = [&]() -> hipError_t {
        const int Is = d->I_shared;
        uint16_t *hs = (uint16_t *)(ws + L.hs);
        float *ys = (float *)(ws + L.ys);
        moe::GemmProblem su{};
        su.mode = up.mode;
        su.A = x;
        su.lda = H;
        su.rows = T;
        su.E = 1;
        su.max_rows = T;
        su.B = w->shared_up;
        su.N = d->act == MOE_ACT_SWIGLU ? 2 * Is : Is;
        su.K = H;
        su.I = Is;
        su.C = hs;
        su.ldc = Is;
        su.limit = up.limit;
        hipError_t err = run(su);
        if (err != hipSuccess)
            return err;
        moe::GemmProblem sd{};
        sd.mode = moe::kDown;
        sd.A = hs;
        sd.lda = Is;
        sd.rows = T;
        sd.E = 1;
        sd.max_rows = T;
        sd.B = w->shared_down;
        sd.N = H;
        sd.K = Is;
        sd.I = Is;
        sd.C = ys;
        sd.ldc = H;
        shared = ys;
        return run(sd);
    };
    if (m > 0) {
        // the segments' rows follow the routed ones: m partial outputs per token
        shared = y + (size_t)A * H;
        shared_terms = m;
    } else if (d->I_shared > 0 && fused) {
        LAUNCH(run_shared());
    }

    if (dq) {
        LAUNCH(moe::launch_dequant(up, wdq, stream));
        LAUNCH(run(dequantized(up)));
    } else {
        LAUNCH(run(up));
    }
    LAUNCH(mark(3));

    if (fused) {
        const moe::CombineArgs comb{slot, wts, shared, shared_terms, T, k, d->routed_scale,
                                    d->fold_routed_scale != 0, out,
                                    d->out_dtype == MOE_OUT_F32};
        LAUNCH(moe::launch_down_combine(down, comb, stream));
    } else if (dq && moe::grouped_supported(dequantized(down))) {
        // (the up projection has read wdq by now: same stream)
        LAUNCH(moe::launch_dequant(down, wdq, stream));
        LAUNCH(run(dequantized(down)));
    } else {
        LAUNCH(run(down));
    }
    LAUNCH(mark(4));

    if (m == 0 && d->I_shared > 0 && !fused)
        LAUNCH(run_shared());
    LAUNCH(mark(5));
    if (!fused)
        LAUNCH(moe::launch_combine(y, slot, wts, shared, shared_terms, T, H, k, d->routed_scale,
                                   d->fold_routed_scale != 0, out,
                                   d->out_dtype == MOE_OUT_F32, stream));
    LAUNCH(mark(6));
    return ok();
}

}  // namespace

int moe_forward(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                void *workspace, size_t workspace_bytes, hipStream_t stream, int32_t *ids_out,
                float *weights_out, int32_t *offsets_out) {
    return forward_impl("moe_forward", d, w, x, out, workspace, workspace_bytes, stream, ids_out,
                        weights_out, offsets_out, nullptr);
}

int moe_forward_profiled(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         int32_t *ids_out, float *weights_out, int32_t *offsets_out,
                         hipEvent_t events[MOE_PROFILE_EVENTS]) {
    return forward_impl("moe_forward_profiled", d, w, x, out, workspace, workspace_bytes, stream,
                        ids_out, weights_out, offsets_out, events);
}

}  // extern "C"

namespace {

// Scratch of moe_forward_noalloc: a file-scope device array, so the entry
// point needs no allocation. Each GPU the library runs on holds its own copy
// (at its own address) until the process ends. In host code `scratch` names
// a host-side stand-in, never the device memory: its device address is
// looked up once per device with hipGetSymbolAddress, and only that address
// is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
int scratch_address(const char *what, void **ptr) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_E_HIP, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
    }
    REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_E_UNSUPPORTED,
            "%s: device %d, need an index below %d", what, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t se = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (se != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(MOE_E_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                        what, dev, hipGetErrorString(se));
        }
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_dims *d, const moe_weights *w, const uint16_t *x, void *out,
                        hipStream_t stream, int32_t *ids_out, float *weights_out,
                        int32_t *offsets_out) {
    const char *what = "moe_forward_noalloc";
    TRY(check_dims(what, d, true));
    const size_t need = layout(*d).total;
    REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_E_WORKSPACE,
            "%s: this call needs %zu bytes of scratch; the static scratch holds %zu "
            "(MOE_NOALLOC_SCRATCH_BYTES): call moe_forward with a workspace instead",
            what, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    if (d->T == 0)      // checks the arguments, enqueues nothing
        return forward_impl(what, d, w, x, out, nullptr, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                            stream, ids_out, weights_out, offsets_out, nullptr, true);
    void *ws = nullptr;
    TRY(scratch_address(what, &ws));
    return forward_impl(what, d, w, x, out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream,
                        ids_out, weights_out, offsets_out, nullptr, true);
}

int moe_add_rmsnorm(int32_t T, int32_t H, const uint16_t *h, const uint16_t *residual,
                    const uint16_t *gamma, float eps, uint16_t *residual_out, uint16_t *x,
                    hipStream_t stream) {
    const char *what = "moe_add_rmsnorm";
    REQUIRE(T >= 0 && T <= (1 << 24), MOE_E_SHAPE, "%s: T = %d, need 0 <= T <= 2^24", what, T);
    REQUIRE(H > 0 && H % 64 == 0 && H <= moe::kNormMaxH, MOE_E_SHAPE,
            "%s: H = %d, need a positive multiple of 64 up to %d", what, H, moe::kNormMaxH);
    REQUIRE(std::isfinite(eps) && eps >= 0.0f, MOE_E_SHAPE, "%s: eps = %g, need a finite value >= 0",
            what, (double)eps);
    if (T == 0)
        return ok();
    TRY(check_opt_ptr(what, "h", h));
    TRY(check_ptr(what, "residual", residual));
    TRY(check_ptr(what, "gamma", gamma));
    TRY(check_opt_ptr(what, "residual_out", residual_out));
    TRY(check_ptr(what, "x", x));
    for (const auto &pr : {std::make_pair("h", (const void *)h),
                           std::make_pair("residual", (const void *)residual),
                           std::make_pair("gamma", (const void *)gamma),
                           std::make_pair("residual_out", (const void *)residual_out),
                           std::make_pair("x", (const void *)x)})
        TRY(check_device(what, pr.first, pr.second));
    LAUNCH(moe::launch_add_rmsnorm(h, residual, gamma, T, H, eps, residual_out, x, stream));
    return ok();
}

const char *moe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
