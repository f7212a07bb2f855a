// C ABI of the compensated block-sparse attention library: argument
// validation on the host, then asynchronous launches on the caller's stream.
#include "../../include/sparse_attn.h"
#include "launch.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sa_status ok() {
    g_last_error.clear();
    return SA_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED(ptr)                                                                          \
    do {                                                                                   \
        if ((ptr) == nullptr) return fail(SA_ERR_INVALID_ARG, "%s must not be NULL", #ptr); \
        if (!aligned(ptr)) return fail(SA_ERR_INVALID_ARG, "%s must be 16-byte aligned", #ptr); \
    } while (0)
#define MAYBE(ptr)                                                                         \
    do {                                                                                   \
        if ((ptr) != nullptr && !aligned(ptr))                                             \
            return fail(SA_ERR_INVALID_ARG, "%s must be 16-byte aligned", #ptr);           \
    } while (0)

static_assert(sa::POOL_STATIC_HEADS == SPARSE_ATTN_POOL_STATIC_HEADS, "static scratch size and header disagree");

constexpr int MAX_BLOCKS = 4096;   // routing keeps one row of keys in LDS; kept-block bitmask size

// Checks the shape; sets `empty` when there is nothing to compute.
sa_status check_shape(const sa_shape* s, bool& empty) {
    if (s == nullptr) return fail(SA_ERR_INVALID_ARG, "shape must not be NULL");
    if (s->B < 0 || s->H < 0 || s->N < 0 || s->N_pad < 0)
        return fail(SA_ERR_INVALID_ARG, "negative size in shape (B=%d H=%d N=%d N_pad=%d)", s->B, s->H, s->N, s->N_pad);
    if (s->d != 64 && s->d != 128) return fail(SA_ERR_INVALID_ARG, "d must be 64 or 128, got %d", s->d);
    const int64_t want = 64 * ((static_cast<int64_t>(s->N) + 63) / 64);
    if (s->N_pad != want)
        return fail(SA_ERR_INVALID_ARG, "N_pad must be 64*ceil(N/64) = %lld, got %d", static_cast<long long>(want), s->N_pad);
    empty = (s->B == 0 || s->H == 0 || s->N == 0);
    return SA_OK;
}

sa_status hip_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* sparse_attn_status_string(sa_status status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported";
        case SA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* sparse_attn_last_error(void) { return g_last_error.c_str(); }

int32_t sparse_attn_abi_version(void) { return SPARSE_ATTN_ABI_VERSION; }

}  // extern "C"

namespace {

// Shared by sparse_attn_pool and sparse_attn_pool_static: the latter passes
// static_ws, and hbar_ws is then the library-owned scratch.
sa_status pool_impl(const sa_shape* shape, sa_dtype dtype, const void* q, const void* k, const void* v,
                    float* qbar, float* kbar, float* vbar, int32_t* kcount, void* cent, void* v16,
                    void* kmom, int8_t* kmom_exp, float* hbar, float* hbar_ws, float* kcov, float* klam,
                    uint8_t* q8, uint8_t* k8, uint8_t* v8, int8_t* exp8, uint8_t* q4, uint8_t* k4,
                    uint8_t* v4, uint8_t* qs4, uint8_t* ks4, uint8_t* vs4, hipStream_t stream, bool static_ws) {
    bool empty = false;
    if (sa_status st = check_shape(shape, empty); st != SA_OK) return st;
    if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (empty) return ok();
    NEED(q); NEED(k); NEED(v); NEED(qbar); NEED(kbar); NEED(vbar); NEED(kcount);
    MAYBE(cent); MAYBE(v16); MAYBE(kmom); MAYBE(hbar); MAYBE(hbar_ws); MAYBE(kcov); MAYBE(klam); MAYBE(q8); MAYBE(k8); MAYBE(v8); MAYBE(exp8);
    MAYBE(q4); MAYBE(k4); MAYBE(v4); MAYBE(qs4); MAYBE(ks4); MAYBE(vs4);
    const int fp4 = (q4 != nullptr) + (k4 != nullptr) + (v4 != nullptr) + (qs4 != nullptr) + (ks4 != nullptr) +
                    (vs4 != nullptr);
    if (fp4 != 0 && fp4 != 6) return fail(SA_ERR_INVALID_ARG, "q4, k4, v4, qs4, ks4 and vs4 must be given together");
    const int fp8 = (q8 != nullptr) + (k8 != nullptr) + (v8 != nullptr) + (exp8 != nullptr);
    if (fp8 != 0 && fp8 != 4) return fail(SA_ERR_INVALID_ARG, "q8, k8, v8 and exp8 must be given together");
    const bool bf16_128 = dtype == SA_BF16 && shape->d == 128;
    if (cent && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "cent needs bf16 inputs with d == 128");
    if (v16 && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "v16 needs bf16 inputs with d == 128");
    if (kmom && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "kmom needs bf16 inputs with d == 128");
    if ((kmom != nullptr) != (kmom_exp != nullptr)) return fail(SA_ERR_INVALID_ARG, "kmom and kmom_exp go together");
    if (!static_ws && (hbar != nullptr) != (hbar_ws != nullptr))
        return fail(SA_ERR_INVALID_ARG, "hbar and hbar_ws go together");
    if (hbar && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "hbar needs bf16 inputs with d == 128");
    if (kcov && !hbar) return fail(SA_ERR_INVALID_ARG, "kcov needs hbar (M_j is taken against H_bar)");
    if (fp8 && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "fp8 copies need bf16 inputs with d == 128");
    if (fp4 && !bf16_128) return fail(SA_ERR_UNSUPPORTED, "MXFP4 copies need bf16 inputs with d == 128");
    if (static_ws && hbar) {
        const int64_t heads = static_cast<int64_t>(shape->B) * shape->H;
        if (heads > sa::POOL_STATIC_HEADS)
            return fail(SA_ERR_UNSUPPORTED, "the library-owned H_bar scratch holds B*H <= %d heads, got %lld",
                        sa::POOL_STATIC_HEADS, static_cast<long long>(heads));
        hbar_ws = sa::pool_static_scratch();
        if (hbar_ws == nullptr) return fail(SA_ERR_HIP, "the library-owned scratch has no address on this device");
    }
    sa::PoolArgs a{shape->B, shape->H, shape->N, shape->N_pad, shape->d, q, k, v, qbar, kbar, vbar, kcount,
                   cent, static_cast<uint16_t*>(v16), kmom, kmom_exp, hbar, hbar_ws, kcov, klam,
                   q8, k8, v8, exp8, q4, k4, v4, qs4, ks4, vs4};
    return hip_result(sa::launch_pool(a, dtype == SA_BF16, stream), "pool");
}

}  // namespace

extern "C" {

sa_status sparse_attn_pool(const sa_shape* shape, sa_dtype dtype, const void* q, const void* k, const void* v,
                           float* qbar, float* kbar, float* vbar, int32_t* kcount, void* cent, void* v16,
                           void* kmom, int8_t* kmom_exp, float* hbar, float* hbar_ws, float* kcov, float* klam,
                           uint8_t* q8, uint8_t* k8, uint8_t* v8, int8_t* exp8, uint8_t* q4, uint8_t* k4,
                           uint8_t* v4, uint8_t* qs4, uint8_t* ks4, uint8_t* vs4, hipStream_t stream) {
    return pool_impl(shape, dtype, q, k, v, qbar, kbar, vbar, kcount, cent, v16, kmom, kmom_exp, hbar, hbar_ws,
                     kcov, klam, q8, k8, v8, exp8, q4, k4, v4, qs4, ks4, vs4, stream, false);
}

sa_status sparse_attn_pool_static(const sa_shape* shape, sa_dtype dtype, const void* q, const void* k,
                                  const void* v, float* qbar, float* kbar, float* vbar, int32_t* kcount,
                                  void* cent, void* v16, void* kmom, int8_t* kmom_exp, float* hbar, float* kcov,
                                  float* klam, uint8_t* q8, uint8_t* k8, uint8_t* v8, int8_t* exp8, uint8_t* q4,
                                  uint8_t* k4, uint8_t* v4, uint8_t* qs4, uint8_t* ks4, uint8_t* vs4,
                                  hipStream_t stream) {
    return pool_impl(shape, dtype, q, k, v, qbar, kbar, vbar, kcount, cent, v16, kmom, kmom_exp, hbar, nullptr,
                     kcov, klam, q8, k8, v8, exp8, q4, k4, v4, qs4, ks4, vs4, stream, true);
}

int32_t sparse_attn_lvsa_capacity(const int32_t* lo, const int32_t* hi, int32_t nb, int32_t window, int32_t anchors) {
    if (lo == nullptr || hi == nullptr || nb <= 0) return 0;
    // window blocks of the widest row plus every anchor (an upper bound over all steps)
    int32_t best = 0;
    for (int a = 0; a < nb; ++a) {
        int32_t c = 0;
        for (int j = 0; j < nb; ++j)
            if (lo[j] <= hi[a] + window && hi[j] >= lo[a] - window) ++c;
        best = c > best ? c : best;
    }
    best += anchors > 0 ? anchors : 0;
    return best > nb ? nb : best;
}

sa_status sparse_attn_route(const sa_shape* shape, const sa_route_spec* spec, const float* qbar, const float* kbar,
                            const int32_t* kcount, const float* kterm, int32_t* idx, int32_t* cnt, int32_t cap,
                            int32_t* idx2, int32_t* cnt2, int32_t cap2, hipStream_t stream) {
    bool empty = false;
    if (sa_status st = check_shape(shape, empty); st != SA_OK) return st;
    if (spec == nullptr) return fail(SA_ERR_INVALID_ARG, "spec must not be NULL");
    const int nb = shape->N_pad / 64;
    if (nb > MAX_BLOCKS) return fail(SA_ERR_UNSUPPORTED, "at most %d blocks per sequence, got %d", MAX_BLOCKS, nb);
    if (empty) return ok();
    sa::RouteArgs a{};
    a.B = shape->B; a.H = shape->H; a.nb = nb; a.d = shape->d; a.N = shape->N; a.mode = spec->mode;
    a.qbar = qbar; a.kbar = kbar; a.kcount = kcount; a.klam = kterm;
    a.idx = idx; a.cnt = cnt; a.cap = cap; a.idx2 = idx2; a.cnt2 = cnt2; a.cap2 = cap2;
    switch (spec->mode) {
        case SA_ROUTE_TOPK:
            NEED(qbar); NEED(kbar); NEED(idx); NEED(cnt);
            if (!empty && (spec->topk < 1 || spec->topk > nb))
                return fail(SA_ERR_INVALID_ARG, "topk must be in [1, nb=%d], got %d", nb, spec->topk);
            if (cap < spec->topk) return fail(SA_ERR_INVALID_ARG, "cap %d < topk %d", cap, spec->topk);
            a.topk = spec->topk;
            break;
        case SA_ROUTE_TOPK_COV:
            NEED(qbar); NEED(kbar); NEED(kterm); NEED(idx); NEED(cnt);
            if (!empty && (spec->topk < 1 || spec->topk > nb))
                return fail(SA_ERR_INVALID_ARG, "topk must be in [1, nb=%d], got %d", nb, spec->topk);
            if (cap < spec->topk) return fail(SA_ERR_INVALID_ARG, "cap %d < topk %d", cap, spec->topk);
            if (!std::isfinite(spec->scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
            a.topk = spec->topk; a.scale = spec->scale;
            break;
        case SA_ROUTE_ERROR:
            NEED(qbar); NEED(kbar); NEED(kcount); NEED(idx); NEED(cnt); NEED(spec->keys); NEED(spec->ekey);
            if (!empty && (spec->topk < 1 || spec->topk > nb))
                return fail(SA_ERR_INVALID_ARG, "topk must be in [1, nb=%d], got %d", nb, spec->topk);
            if (cap < spec->topk) return fail(SA_ERR_INVALID_ARG, "cap %d < topk %d", cap, spec->topk);
            if (!std::isfinite(spec->scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
            if (shape->d != 128) return fail(SA_ERR_UNSUPPORTED, "error-aware routing supports d == 128 only");
            a.topk = spec->topk; a.scale = spec->scale; a.keys = spec->keys; a.ekey = spec->ekey;
            break;
        case SA_ROUTE_LVSA:
            NEED(spec->frame_lo); NEED(spec->frame_hi); NEED(idx); NEED(cnt);
            if (spec->window < 0 || spec->anchor_phase < 0 || spec->step < 0)
                return fail(SA_ERR_INVALID_ARG, "window, anchor_phase and step must be >= 0");
            if (spec->anchors < 0 || (!empty && spec->anchors > nb))
                return fail(SA_ERR_INVALID_ARG, "anchors must be in [0, nb=%d], got %d", nb, spec->anchors);
            if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
            a.frame_lo = spec->frame_lo; a.frame_hi = spec->frame_hi; a.window = spec->window;
            a.anchors = spec->anchors; a.anchor_phase = spec->anchor_phase; a.step = spec->step;
            break;
        case SA_ROUTE_TRIAGE:
            NEED(qbar); NEED(kbar); NEED(kcount); NEED(kterm); NEED(cnt);
            if (!empty && (spec->n_keep < 1 || spec->n_keep > nb))
                return fail(SA_ERR_INVALID_ARG, "n_keep must be in [1, nb=%d], got %d", nb, spec->n_keep);
            if (spec->n_refine < 0 || spec->n_refine > spec->n_keep)
                return fail(SA_ERR_INVALID_ARG, "n_refine must be in [0, n_keep], got %d", spec->n_refine);
            if (cap < spec->n_refine) return fail(SA_ERR_INVALID_ARG, "cap %d < n_refine %d", cap, spec->n_refine);
            if (cap > 0) NEED(idx); else MAYBE(idx);
            if (cap2 < spec->n_keep - spec->n_refine)
                return fail(SA_ERR_INVALID_ARG, "cap2 %d < n_keep - n_refine %d", cap2, spec->n_keep - spec->n_refine);
            NEED(cnt2);
            if (cap2 > 0) NEED(idx2); else MAYBE(idx2);
            if (!std::isfinite(spec->scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
            a.n_keep = spec->n_keep; a.n_refine = spec->n_refine; a.scale = spec->scale;
            break;
        default:
            return fail(SA_ERR_INVALID_ARG, "unknown route mode %d", spec->mode);
    }
    if (empty) return ok();
    return hip_result(sa::launch_route(a, stream), "route");
}

size_t sparse_attn_residual_workspace(const sa_shape* shape) {
    if (shape == nullptr || shape->B < 0 || shape->H < 0 || shape->N_pad < 0) return 0;
    return sa::residual_workspace_bytes(shape->B, shape->H, shape->N_pad);
}

sa_status sparse_attn_residual(const sa_shape* shape, sa_dtype dtype, float scale, const void* q, const void* k,
                               const void* v, void* out, int32_t phase, float ridge, int32_t rank, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    bool empty = false;
    if (sa_status st = check_shape(shape, empty); st != SA_OK) return st;
    if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "the residual pass takes bf16 tensors");
    if (shape->d != 128) return fail(SA_ERR_UNSUPPORTED, "the residual pass supports d == 128 only");
    const int nb = shape->N_pad / 64;
    if (nb > MAX_BLOCKS) return fail(SA_ERR_UNSUPPORTED, "at most %d blocks per sequence, got %d", MAX_BLOCKS, nb);
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(SA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (!std::isfinite(ridge) || ridge < 0.0f) return fail(SA_ERR_INVALID_ARG, "ridge must be finite and >= 0");
    if (rank < 1 || rank > 8) return fail(SA_ERR_INVALID_ARG, "rank must be in [1, 8], got %d", rank);
    if (phase < 0) return fail(SA_ERR_INVALID_ARG, "phase must be >= 0");
    if (empty) return ok();
    NEED(q); NEED(k); NEED(v); NEED(out); NEED(workspace);
    const size_t need = sa::residual_workspace_bytes(shape->B, shape->H, shape->N_pad);
    if (workspace_bytes < need)
        return fail(SA_ERR_INVALID_ARG, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    sa::ResidualArgs r{};
    r.B = shape->B; r.H = shape->H; r.N = shape->N; r.N_pad = shape->N_pad;
    r.Mp = 64 * ((nb + 63) / 64);
    r.phase = phase; r.rank = rank; r.scale = scale; r.ridge = ridge;
    r.q = q; r.k = k; r.v = v; r.out = out;
    sa::residual_carve(r, workspace);
    return hip_result(sa::launch_residual(r, stream), "residual");
}

sa_status sparse_attn_fwd(const sa_shape* shape, sa_dtype dtype, sa_comp comp, float scale, const void* q,
                          const void* k, const void* v, const float* kbar, const float* vbar, const void* cent,
                          const void* v16, const int32_t* kcount, const void* kmom, const int8_t* kmom_exp,
                          const float* hbar, const uint8_t* q8,
                          const uint8_t* k8, const uint8_t* v8,
                          const int8_t* exp8, sa_skim_format skim_fmt, const uint8_t* q4, const uint8_t* k4,
                          const uint8_t* v4, const uint8_t* qs4, const uint8_t* ks4, const uint8_t* vs4,
                          const int32_t* idx, const int32_t* cnt, int32_t cap,
                          const int32_t* idx2, const int32_t* cnt2, int32_t cap2, void* out, float* lse,
                          hipStream_t stream) {
    bool empty = false;
    if (sa_status st = check_shape(shape, empty); st != SA_OK) return st;
    if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (comp < SA_COMP_DROP || comp > SA_COMP_ORDER1_GLOBAL)
        return fail(SA_ERR_INVALID_ARG, "unknown compensation order %d", static_cast<int>(comp));
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(SA_ERR_INVALID_ARG, "scale must be finite and > 0");
    const int nb = shape->N_pad / 64;
    if (nb > MAX_BLOCKS) return fail(SA_ERR_UNSUPPORTED, "at most %d blocks per sequence, got %d", MAX_BLOCKS, nb);
    if (empty) return ok();
    NEED(q); NEED(k); NEED(v); NEED(out); MAYBE(lse); MAYBE(kbar); MAYBE(vbar); MAYBE(cent); MAYBE(v16);
    if (cap < 0 || cap2 < 0) return fail(SA_ERR_INVALID_ARG, "cap and cap2 must be >= 0");
    if (cap > 0) { NEED(idx); NEED(cnt); }
    const bool skim = idx2 != nullptr && cap2 > 0;
    if (skim) { NEED(cnt2); }
    if (comp >= SA_COMP_ORDER0) { NEED(kcount); }
    if (comp == SA_COMP_ORDER1_BLOCK) { NEED(kmom); NEED(kmom_exp); }
    if (comp == SA_COMP_ORDER1_GLOBAL) { NEED(hbar); }
    if (dtype == SA_F32) {
        if (comp >= SA_COMP_ORDER0) { NEED(kbar); NEED(vbar); }
        if (shape->d != 64) return fail(SA_ERR_UNSUPPORTED, "fp32 forward supports d == 64 only");
        if (comp >= SA_COMP_ORDER1_BLOCK) return fail(SA_ERR_UNSUPPORTED, "fp32 forward has no first-order term");
        if (skim) return fail(SA_ERR_UNSUPPORTED, "fp32 forward has no fp8 skim tier");
    } else {
        if (shape->d != 128) return fail(SA_ERR_UNSUPPORTED, "bf16 forward supports d == 128 only");
        NEED(v16);
        if (comp >= SA_COMP_ORDER0) { NEED(cent); }
        if (skim && skim_fmt == SA_SKIM_E4M3) { NEED(q8); NEED(k8); NEED(v8); NEED(exp8); }
        if (skim && skim_fmt == SA_SKIM_MXFP4) { NEED(q4); NEED(k4); NEED(v4); NEED(qs4); NEED(ks4); NEED(vs4); }
    }
    if (skim_fmt != SA_SKIM_E4M3 && skim_fmt != SA_SKIM_MXFP4)
        return fail(SA_ERR_INVALID_ARG, "unknown skim format %d", static_cast<int>(skim_fmt));
    if (comp == SA_COMP_DROP && cap == 0 && !skim)
        return fail(SA_ERR_INVALID_ARG, "drop mode needs exact or skim lists");
    sa::FwdArgs a{shape->B, shape->H, shape->N, shape->N_pad, shape->d, static_cast<int>(comp), scale, q, k, v,
                  kbar, vbar, cent, v16, kcount, kmom, kmom_exp, hbar, q8, k8, v8, exp8, q4, k4, v4, qs4, ks4, vs4,
                  static_cast<int>(skim_fmt), idx, cnt, cap, idx2, cnt2, cap2, out, lse,
                  shape->N, shape->N_pad, 0, 0};
    if (dtype == SA_F32) return hip_result(sa::launch_fwd_f32(a, stream), "fwd_f32");
    return hip_result(sa::launch_fwd_bf16(a, stream), "fwd_bf16");
}

}  // extern "C"
