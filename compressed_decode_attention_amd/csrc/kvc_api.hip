// kvc_api.hip -- the extern "C" entry points of libkvc: host-side argument
// validation (nothing is enqueued when a call fails), workspace layout,
// split selection and kernel dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kvc_internal.h"

#define KVC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

kvc_status fail(kvc_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
kvc_status fail(kvc_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

kvc_status ok() {
    g_err[0] = '\0';
    return KVC_OK;
}

constexpr size_t kAlign = 256;
constexpr int kMaxUnits = 1 << 24;   // sequences x kv heads in one call
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

kvc_status check_cache(const kvc_cache *c, const char *what) {
    if (!c) return fail(KVC_ERR_INVALID_ARG, "%s: cache is NULL", what);
    if (c->batch <= 0 || c->q_heads <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 ||
        c->capacity <= 0)
        return fail(KVC_ERR_INVALID_ARG, "%s: batch, heads, head_dim and capacity must be > 0",
                    what);
    if (c->q_heads % c->kv_heads != 0)
        return fail(KVC_ERR_SHAPE, "%s: q_heads %d is not a multiple of kv_heads %d", what,
                    c->q_heads, c->kv_heads);
    if (c->q_heads / c->kv_heads > kvc::kMaxGroup)
        return fail(KVC_ERR_UNSUPPORTED, "%s: group size %d > %d", what,
                    c->q_heads / c->kv_heads, kvc::kMaxGroup);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(KVC_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", what, c->head_dim);
    if (c->dtype != KVC_BF16 && c->dtype != KVC_F32 && c->dtype != KVC_FP8_E5M2)
        return fail(KVC_ERR_UNSUPPORTED, "%s: dtype %d", what, c->dtype);
    if (c->capacity > kvc::kMaxCapacity)
        return fail(KVC_ERR_UNSUPPORTED, "%s: capacity %d > %d", what, c->capacity,
                    kvc::kMaxCapacity);
    // launches are one workgroup per unit times at most 64 splits: the grid
    // stays below 2^31 workgroups
    if ((int64_t)c->batch * c->kv_heads > kMaxUnits)
        return fail(KVC_ERR_UNSUPPORTED, "%s: batch x kv_heads = %lld units > %d", what,
                    (long long)c->batch * c->kv_heads, kMaxUnits);
    if (!c->k || !c->v || !c->pos || !c->n_slots)
        return fail(KVC_ERR_INVALID_ARG, "%s: k, v, pos and n_slots must not be NULL", what);
    if ((uintptr_t)c->k % 16 || (uintptr_t)c->v % 16)
        return fail(KVC_ERR_INVALID_ARG, "%s: k and v must be 16-byte aligned", what);
    if (c->block_size < 0)
        return fail(KVC_ERR_INVALID_ARG, "%s: block_size < 0", what);
    if (c->block_size > 0) {
        if (!c->block_table)
            return fail(KVC_ERR_INVALID_ARG, "%s: paged cache without block_table", what);
        if (c->max_blocks <= 0 || c->num_blocks <= 0)
            return fail(KVC_ERR_SHAPE, "%s: max_blocks and num_blocks must be > 0", what);
        if ((int64_t)c->max_blocks * c->block_size != c->capacity)
            return fail(KVC_ERR_SHAPE, "%s: capacity %d != max_blocks %d x block_size %d", what,
                        c->capacity, c->max_blocks, c->block_size);
    }
    return KVC_OK;
}

int units_of(const kvc_cache *c) { return c->batch * c->kv_heads; }

// Workgroups per unit for a unit length of up to `hint` attended entries:
// at most 1024 keys per workgroup, and enough workgroups to cover the chip
// when the batch is small (never below 256 keys per workgroup).
int choose_nsplit(const kvc_cache *c, int hint) {
    const int T = (hint <= 0 || hint > c->capacity + 1) ? c->capacity + 1 : hint;
    const int units = units_of(c);
    if (kvc::mfma_tiles_ok(c->dtype, c->head_dim, c->block_size) && T > kvc::kFusedMaxT) {
        // matrix-core splits: chunks of at most 528 slots (the 528-entry LDS
        // instance, four workgroups per CU), and at least about 2,048
        // workgroups in all (two per resident slot) while no chunk falls
        // under 128 slots; at most 64 splits.  Longer chunks are cheaper per
        // byte: at 256 units of 5,121 slots, 10 splits step in 121 us where
        // 16 take 133 us and 20 take 148 us.
        int ns = (T + 527) / 528;
        const int fill = (2048 + units - 1) / units, by_len = (T + 127) / 128;
        const int want = fill < by_len ? fill : by_len;
        ns = ns > want ? ns : want;
        return ns > 64 ? 64 : ns;
    }
    int ns = (T + 1023) / 1024;
    if (units < 2048) {
        int fill = (2048 + units - 1) / units;
        int by_len = (T + 255) / 256;
        fill = fill < by_len ? fill : by_len;
        ns = ns > fill ? ns : fill;
    }
    if (ns < 1) ns = 1;
    if (ns > 64) ns = 64;
    return ns;
}

// Attended length the caller promises (n_slots + 1 <= hint); <= 0 means the
// capacity bound.
int effective_len(const kvc_cache *c, int hint) {
    return (hint <= 0 || hint > c->capacity + 1) ? c->capacity + 1 : hint;
}

bool use_fused(const kvc_cache *c, int hint) {
    // paged: power-of-two blocks of at least one 16-slot tile
    const bool tile_blocks = c->block_size == 0 ||
                             (c->block_size >= 16 && (c->block_size & (c->block_size - 1)) == 0);
    return (c->dtype == KVC_BF16 || c->dtype == KVC_FP8_E5M2) && c->head_dim == 128 && tile_blocks &&
           effective_len(c, hint) <= kvc::kFusedMaxT;
}

struct Workspace {
    size_t part_off, part_bytes;
    size_t logit_off, logit_bytes;
    size_t keep_off, keep_bytes;
    size_t nout_off, nout_bytes;
    size_t presel_off, presel_bytes;
    size_t order_off, order_bytes;
    size_t total;
    int nsplit;
    int max_len;   // attended length bound of every unit
};

Workspace layout(const kvc_cache *c, int hint) {
    Workspace w;
    const size_t units = (size_t)units_of(c);
    const size_t G = (size_t)(c->q_heads / c->kv_heads);
    w.nsplit = choose_nsplit(c, hint);
    w.max_len = effective_len(c, hint);
    w.part_bytes = w.nsplit > 1 ? units * w.nsplit * G * (c->head_dim + 2) * sizeof(float) : 0;
    w.logit_bytes = units * G * ((size_t)c->capacity + 1) * sizeof(float);
    w.keep_bytes = units * (size_t)c->capacity * sizeof(int32_t);
    w.nout_bytes = units * sizeof(int32_t);
    w.presel_bytes =
        w.nsplit > 1 ? units * w.nsplit * kvc::kPreselWaves * sizeof(kvc::PreselRecord) : 0;
    size_t off = 0;
    w.part_off = off;
    off += align_up(w.part_bytes);
    w.logit_off = off;
    off += align_up(w.logit_bytes);
    w.keep_off = off;
    off += align_up(w.keep_bytes);
    w.nout_off = off;
    off += align_up(w.nout_bytes);
    w.presel_off = off;
    off += align_up(w.presel_bytes);
    w.order_bytes = w.nsplit > 1 ? units * sizeof(int32_t) : 0;
    w.order_off = off;
    off += align_up(w.order_bytes);
    w.total = off;
    return w;
}

kvc_status check_ws(const Workspace &w, void *ws, size_t bytes, const char *what) {
    if (w.total == 0) return KVC_OK;
    if (!ws) return fail(KVC_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", what, w.total);
    if (bytes < w.total)
        return fail(KVC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what, bytes, w.total);
    if ((uintptr_t)ws % kAlign)
        return fail(KVC_ERR_WORKSPACE, "%s: workspace must be %zu-byte aligned", what, kAlign);
    return KVC_OK;
}

kvc_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

kvc_status check_policy(const kvc_policy *p, const float *scores, const char *what) {
    if (!p) return fail(KVC_ERR_INVALID_ARG, "%s: policy is NULL", what);
    switch (p->kind) {
        case KVC_POLICY_FULL:
            return KVC_OK;
        case KVC_POLICY_STREAMING:
            if (p->n_sink < 0 || p->n_recent < 0)
                return fail(KVC_ERR_INVALID_ARG, "%s: n_sink and n_recent must be >= 0", what);
            return KVC_OK;
        case KVC_POLICY_H2O:
            if (p->n_heavy < 0 || p->n_recent < 0)
                return fail(KVC_ERR_INVALID_ARG, "%s: n_heavy and n_recent must be >= 0", what);
            if (!scores) return fail(KVC_ERR_INVALID_ARG, "%s: H2O needs h2o_scores", what);
            if (!(p->decay >= 0.f && p->decay < 1.f))
                return fail(KVC_ERR_INVALID_ARG, "%s: decay must be 0 or in (0, 1)", what);
            return KVC_OK;
        case KVC_POLICY_RANDOM:
            if (p->prompt_len < 0 || p->n_keep < 0)
                return fail(KVC_ERR_INVALID_ARG, "%s: prompt_len and n_keep must be >= 0", what);
            return KVC_OK;
        default:
            return fail(KVC_ERR_INVALID_ARG, "%s: unknown policy kind %d", what, p->kind);
    }
}

kvc::AttnArgs attn_args(const kvc_cache *c, const int32_t *new_pos, const void *q,
                        const void *k_new, const void *v_new, float *out, float *scores,
                        float scale, float decay, const Workspace &w, void *ws) {
    kvc::AttnArgs a;
    a.c = kvc::make_dev(*c);
    a.decay = decay;
    a.new_pos = new_pos;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.out = out;
    a.scores = scores;
    a.scale = scale;
    a.nsplit = w.nsplit;
    a.max_len = w.max_len;
    a.append = true;
    a.part = w.part_bytes ? (float *)((char *)ws + w.part_off) : nullptr;
    a.logits = (float *)((char *)ws + w.logit_off);
    a.order = w.order_bytes ? (int32_t *)((char *)ws + w.order_off) : nullptr;
    return a;
}

// Arguments of the one-workgroup-per-unit kernel; its fallback routines use
// the same workspace regions as the split path (logits, keep lists).
kvc::FusedArgs fused_args(const kvc_cache *c, const kvc::AttnArgs &a, int hint) {
    kvc::FusedArgs fa;
    fa.attn = a;
    fa.attn.nsplit = 1;
    fa.attn.part = nullptr;
    fa.tcap = effective_len(c, hint) <= kvc::kFusedSmallT ? kvc::kFusedSmallT : kvc::kFusedMaxT;
    fa.sel = kvc::SelectArgs();
    fa.comp = kvc::CompactArgs();
    fa.e5m2 = c->dtype == KVC_FP8_E5M2;
    return fa;
}

kvc_status check_attn_args(const kvc_cache *c, const int32_t *new_pos, const void *q,
                           const void *k_new, const void *v_new, const float *out, float scale,
                           const char *what) {
    kvc_status s = check_cache(c, what);
    if (s != KVC_OK) return s;
    if (!new_pos || !q || !k_new || !v_new || !out)
        return fail(KVC_ERR_INVALID_ARG, "%s: new_pos, q, k_new, v_new and out must not be NULL",
                    what);
    if (!isfinite(scale)) return fail(KVC_ERR_INVALID_ARG, "%s: scale is not finite", what);
    // the matrix-core kernels read q, k_new and v_new and write out in
    // 16-byte pieces
    if ((uintptr_t)q % 16 || (uintptr_t)k_new % 16 || (uintptr_t)v_new % 16 || (uintptr_t)out % 16)
        return fail(KVC_ERR_INVALID_ARG, "%s: q, k_new, v_new and out must be 16-byte aligned",
                    what);
    return KVC_OK;
}

kvc::SelectArgs select_args(const kvc_cache *c, const kvc_policy &p, uint32_t step,
                            const float *scores, int32_t *keep, int32_t *nout) {
    kvc::SelectArgs a;
    a.c = kvc::make_dev(*c);
    a.kind = p.kind;
    a.n_sink = p.n_sink;
    a.n_heavy = p.n_heavy;
    a.n_recent = p.n_recent;
    a.prompt_len = p.prompt_len;
    a.n_keep = p.n_keep;
    a.seed = p.seed;
    a.step = step;
    a.scores = scores;
    a.keep_slots = keep;
    a.n_out = nout;
    return a;
}

}  // namespace

// ---------------------------------------------------------------------------

KVC_EXPORT size_t kvc_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                      int32_t dtype_bytes) {
    if (layers <= 0 || kv_heads <= 0 || head_dim <= 0 || dtype_bytes <= 0) return 0;
    return (size_t)2 * (size_t)layers * (size_t)kv_heads * (size_t)head_dim * (size_t)dtype_bytes;
}

KVC_EXPORT int64_t kvc_n_keep(int64_t n_candidates, double keep_ratio) {
    if (n_candidates <= 0) return 0;
    const double prod = (double)n_candidates * keep_ratio;
    int64_t k = (prod >= 9.2e18) ? n_candidates : (int64_t)prod;   // truncation toward zero
    if (k < 1) k = 1;
    if (k > n_candidates) k = n_candidates;
    return k;
}

KVC_EXPORT const char *kvc_status_string(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_INVALID_ARG: return "invalid argument";
        case KVC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case KVC_ERR_SHAPE: return "inconsistent shapes";
        case KVC_ERR_WORKSPACE: return "workspace missing or too small";
        case KVC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

KVC_EXPORT const char *kvc_last_error(void) { return g_err; }

KVC_EXPORT size_t kvc_workspace_bytes(const kvc_cache *c, int32_t max_len_hint) {
    if (check_cache(c, "kvc_workspace_bytes") != KVC_OK) return 0;
    return layout(c, max_len_hint).total;
}

KVC_EXPORT kvc_status kvc_decode_attn(const kvc_cache *c, const int32_t *new_pos, const void *q,
                                      const void *k_new, const void *v_new, float *out,
                                      float *h2o_scores, float scale, float score_decay,
                                      int32_t max_len_hint, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    const char *what = "kvc_decode_attn";
    kvc_status s = check_attn_args(c, new_pos, q, k_new, v_new, out, scale, what);
    if (s != KVC_OK) return s;
    if (!(score_decay >= 0.f && score_decay < 1.f))
        return fail(KVC_ERR_INVALID_ARG, "%s: score_decay must be 0 or in (0, 1)", what);
    const Workspace w = layout(c, max_len_hint);
    if ((s = check_ws(w, workspace, workspace_bytes, what)) != KVC_OK) return s;
    kvc::AttnArgs a = attn_args(c, new_pos, q, k_new, v_new, out, h2o_scores, scale,
                                h2o_scores ? score_decay : 0.f, w, workspace);
    if (use_fused(c, max_len_hint)) {
        kvc::FusedArgs fa = fused_args(c, a, max_len_hint);
        return hip_status(kvc::launch_fused(fa, kvc::kModeAttn, (hipStream_t)stream), what);
    }
    return hip_status(kvc::launch_attn(a, c->dtype, (hipStream_t)stream), what);
}

// the matrix-core prompt scoring: bf16 K, head_dim 128, and a sequence's
// query rows and a unit's K rows each within the 2 GiB its buffer loads address
static bool use_prompt_mfma(const kvc_cache *c, int32_t m_rows) {
    const size_t limit = (size_t)1 << 31;
    return c->dtype == KVC_BF16 && c->head_dim == 128 &&
           (size_t)m_rows * (size_t)c->q_heads * 256 < limit && (size_t)c->capacity * 256 < limit;
}

KVC_EXPORT size_t kvc_h2o_accumulate_workspace_bytes(const kvc_cache *c, int32_t m_rows) {
    if (check_cache(c, "kvc_h2o_accumulate_workspace_bytes") != KVC_OK || m_rows <= 0) return 0;
    if (!use_prompt_mfma(c, m_rows)) return 0;
    return align_up(kvc::prompt_workspace_bytes(c->batch * c->kv_heads, m_rows,
                                                c->q_heads / c->kv_heads));
}

KVC_EXPORT kvc_status kvc_h2o_accumulate(const kvc_cache *c, const void *q_rows, int32_t m_rows,
                                         const int32_t *q_pos, float *h2o_scores, float scale,
                                         void *workspace, size_t workspace_bytes,
                                         void *stream) {
    const char *what = "kvc_h2o_accumulate";
    kvc_status s = check_cache(c, what);
    if (s != KVC_OK) return s;
    if (m_rows < 0) return fail(KVC_ERR_INVALID_ARG, "%s: m_rows < 0", what);
    if (m_rows == 0) return ok();
    if (!q_rows || !h2o_scores)
        return fail(KVC_ERR_INVALID_ARG, "%s: q_rows and h2o_scores must not be NULL", what);
    if (!isfinite(scale)) return fail(KVC_ERR_INVALID_ARG, "%s: scale is not finite", what);
    if (use_prompt_mfma(c, m_rows)) {
        if ((uintptr_t)q_rows % 16)
            return fail(KVC_ERR_INVALID_ARG, "%s: q_rows must be 16-byte aligned", what);
        Workspace w{};
        w.total = kvc_h2o_accumulate_workspace_bytes(c, m_rows);
        if ((s = check_ws(w, workspace, workspace_bytes, what)) != KVC_OK) return s;
        kvc::PromptArgs p;
        p.c = kvc::make_dev(*c);
        p.q_rows = q_rows;
        p.m_rows = m_rows;
        p.q_pos = q_pos;
        p.scores = h2o_scores;
        p.scale = scale;
        p.lse = static_cast<float *>(workspace);
        return hip_status(kvc::launch_prompt_scores(p, (hipStream_t)stream), what);
    }
    kvc::AccumArgs a;
    a.c = kvc::make_dev(*c);
    a.q_rows = q_rows;
    a.m_rows = m_rows;
    a.q_pos = q_pos;
    a.scores = h2o_scores;
    a.scale = scale;
    return hip_status(kvc::launch_accumulate(a, c->dtype, (hipStream_t)stream), what);
}

static kvc_status evict_common(const char *what, const kvc_cache *c, const kvc_policy &p,
                               uint32_t step, const float *scores, int32_t *keep_slots,
                               int32_t *n_out, void *stream) {
    kvc_status s = check_cache(c, what);
    if (s != KVC_OK) return s;
    if ((s = check_policy(&p, scores, what)) != KVC_OK) return s;
    if (!keep_slots || !n_out)
        return fail(KVC_ERR_INVALID_ARG, "%s: keep_slots and n_out must not be NULL", what);
    kvc::SelectArgs a = select_args(c, p, step, scores, keep_slots, n_out);
    return hip_status(kvc::launch_select(a, (hipStream_t)stream), what);
}

KVC_EXPORT kvc_status kvc_evict_streaming(const kvc_cache *c, int32_t n_sink, int32_t n_recent,
                                          int32_t *keep_slots, int32_t *n_out, void *stream) {
    kvc_policy p = {};
    p.kind = KVC_POLICY_STREAMING;
    p.n_sink = n_sink;
    p.n_recent = n_recent;
    return evict_common("kvc_evict_streaming", c, p, 0, nullptr, keep_slots, n_out, stream);
}

KVC_EXPORT kvc_status kvc_evict_h2o(const kvc_cache *c, const float *h2o_scores, int32_t n_heavy,
                                    int32_t n_recent, int32_t *keep_slots, int32_t *n_out,
                                    void *stream) {
    kvc_policy p = {};
    p.kind = KVC_POLICY_H2O;
    p.n_heavy = n_heavy;
    p.n_recent = n_recent;
    return evict_common("kvc_evict_h2o", c, p, 0, h2o_scores, keep_slots, n_out, stream);
}

KVC_EXPORT kvc_status kvc_evict_random(const kvc_cache *c, int32_t prompt_len, int32_t n_keep,
                                       uint64_t seed, uint32_t step, int32_t *keep_slots,
                                       int32_t *n_out, void *stream) {
    kvc_policy p = {};
    p.kind = KVC_POLICY_RANDOM;
    p.prompt_len = prompt_len;
    p.n_keep = n_keep;
    p.seed = seed;
    return evict_common("kvc_evict_random", c, p, step, nullptr, keep_slots, n_out, stream);
}

KVC_EXPORT kvc_status kvc_compact(const kvc_cache *c, const int32_t *keep_slots,
                                  const int32_t *n_out, float *h2o_scores,
                                  const kvc_cache *ordered_dst, void *stream) {
    const char *what = "kvc_compact";
    kvc_status s = check_cache(c, what);
    if (s != KVC_OK) return s;
    if (!keep_slots || !n_out)
        return fail(KVC_ERR_INVALID_ARG, "%s: keep_slots and n_out must not be NULL", what);
    kvc::CompactArgs a;
    a.c = kvc::make_dev(*c);
    a.keep_slots = keep_slots;
    a.n_out = n_out;
    a.scores = h2o_scores;
    a.ordered = ordered_dst != nullptr;
    if (ordered_dst) {
        if ((s = check_cache(ordered_dst, what)) != KVC_OK) return s;
        if (ordered_dst->batch != c->batch || ordered_dst->q_heads != c->q_heads ||
            ordered_dst->kv_heads != c->kv_heads || ordered_dst->head_dim != c->head_dim ||
            ordered_dst->dtype != c->dtype)
            return fail(KVC_ERR_SHAPE, "%s: ordered_dst shape or dtype differs from the cache",
                        what);
        if (ordered_dst->k == c->k || ordered_dst->v == c->v)
            return fail(KVC_ERR_INVALID_ARG, "%s: ordered_dst must not alias the cache", what);
        a.dst = kvc::make_dev(*ordered_dst);
    } else {
        a.dst = a.c;
    }
    return hip_status(kvc::launch_compact(a, c->dtype, (hipStream_t)stream), what);
}

static kvc_status decode_step(const char *what, const kvc_cache *c, const kvc_policy *policy,
                              uint32_t step, const int32_t *new_pos, const void *q,
                              const void *k_new, const void *v_new, float *out,
                              float *h2o_scores, float scale, int32_t max_len_hint,
                              void *workspace, size_t workspace_bytes, void *stream) {
    kvc_status s = check_attn_args(c, new_pos, q, k_new, v_new, out, scale, what);
    if (s != KVC_OK) return s;
    if ((s = check_policy(policy, h2o_scores, what)) != KVC_OK) return s;
    const Workspace w = layout(c, max_len_hint);
    if ((s = check_ws(w, workspace, workspace_bytes, what)) != KVC_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    float *scores = policy->kind == KVC_POLICY_H2O ? h2o_scores : nullptr;
    kvc::AttnArgs a = attn_args(c, new_pos, q, k_new, v_new, out, scores, scale,
                                scores ? policy->decay : 0.f, w, workspace);
    int32_t *keep = (int32_t *)((char *)workspace + w.keep_off);
    int32_t *nout = (int32_t *)((char *)workspace + w.nout_off);
    kvc::SelectArgs sa = select_args(c, *policy, step, scores, keep, nout);
    if (use_fused(c, max_len_hint)) {
        kvc::FusedArgs fa = fused_args(c, a, max_len_hint);
        fa.sel = sa;
        fa.comp.c = kvc::make_dev(*c);
        fa.comp.keep_slots = keep;
        fa.comp.n_out = nout;
        fa.comp.scores = scores;
        fa.comp.ordered = false;
        fa.comp.dst = fa.comp.c;
        return hip_status(kvc::launch_fused(fa, kvc::kModeStep, st), what);
    }
    if (policy->kind == KVC_POLICY_FULL)
        return hip_status(kvc::launch_attn(a, c->dtype, st), what);
    kvc::CompactArgs ca;
    ca.c = kvc::make_dev(*c);
    ca.keep_slots = keep;
    ca.n_out = nout;
    ca.scores = scores;
    ca.ordered = false;
    ca.dst = ca.c;
    if (policy->kind == KVC_POLICY_RANDOM && a.nsplit > 1 &&
        kvc::mfma_tiles_ok(c->dtype, c->head_dim, c->block_size)) {
        // the matrix-core split kernels rank their own chunks' candidates
        a.presel = (uint32_t *)((char *)workspace + w.presel_off);
        a.presel_prompt_len = policy->prompt_len;
        a.presel_step = step;
        a.presel_seed = policy->seed;
    }
    return hip_status(kvc::launch_step_split(a, sa, ca, c->dtype, st), what);
}

KVC_EXPORT kvc_status kvc_decode_step(const kvc_cache *c, const kvc_policy *policy, uint32_t step,
                                      const int32_t *new_pos, const void *q, const void *k_new,
                                      const void *v_new, float *out, float *h2o_scores,
                                      float scale, int32_t max_len_hint, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    return decode_step("kvc_decode_step", c, policy, step, new_pos, q, k_new, v_new, out,
                       h2o_scores, scale, max_len_hint, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// kvc_decode_step without a caller workspace: the same kernels take their
// scratch (split partials, fallback logits, keep lists) from one static
// device array of KVC_NOALLOC_SCRATCH_BYTES.  Host code never passes the
// array's name to a kernel (in host code it names a host-side stand-in): the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is used.  Nothing in the scratch has to start at zero (every
// region is written before it is read within a call), so no clearing is
// enqueued.  Calls on one device share the array: calls that overlap on one
// GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on the current device (looked up once).
kvc_status scratch_of_current_device(void **ptr, const char *what) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVC_ERR_HIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVC_ERR_UNSUPPORTED, "%s: device %d beyond %d", what, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVC_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", what,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KVC_OK;
}
}  // namespace

KVC_EXPORT kvc_status kvc_decode_step_noalloc(const kvc_cache *c, const kvc_policy *policy,
                                              uint32_t step, const int32_t *new_pos,
                                              const void *q, const void *k_new,
                                              const void *v_new, float *out, float *h2o_scores,
                                              float scale, int32_t max_len_hint, void *stream) {
    const char *what = "kvc_decode_step_noalloc";
    // every argument and the scratch size are checked before the device is touched
    kvc_status s = check_attn_args(c, new_pos, q, k_new, v_new, out, scale, what);
    if (s != KVC_OK) return s;
    if ((s = check_policy(policy, h2o_scores, what)) != KVC_OK) return s;
    const size_t need = layout(c, max_len_hint).total;
    if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES)
        return fail(KVC_ERR_WORKSPACE,
                    "%s: this cache and length hint need %zu bytes of scratch; the static "
                    "scratch holds %zu (use kvc_decode_step with a workspace)",
                    what, need, (size_t)KVC_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((s = scratch_of_current_device(&ws, what)) != KVC_OK) return s;
    return decode_step(what, c, policy, step, new_pos, q, k_new, v_new, out, h2o_scores, scale,
                       max_len_hint, ws, (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream);
}

KVC_EXPORT kvc_status kvc_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                      void *stream) {
    const char *what = "kvc_stream_read";
    if (!src || !sink) return fail(KVC_ERR_INVALID_ARG, "%s: src and sink must not be NULL", what);
    if ((uintptr_t)src % 16 || bytes == 0 || bytes % 16)
        return fail(KVC_ERR_INVALID_ARG,
                    "%s: src must be 16-byte aligned and bytes a positive multiple of 16", what);
    return hip_status(kvc::launch_stream_read(src, bytes, sink, (hipStream_t)stream), what);
}

// ---------------------------------------------------------------------------
// KIVI-style quantized cache
// ---------------------------------------------------------------------------
namespace {

kvc_status check_kivi(const kvc_kivi_cache *c, const char *what) {
    if (!c) return fail(KVC_ERR_INVALID_ARG, "%s: cache is NULL", what);
    if (c->batch <= 0 || c->q_heads <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 ||
        c->max_quant < 0)
        return fail(KVC_ERR_INVALID_ARG, "%s: batch, heads, head_dim must be > 0, max_quant >= 0",
                    what);
    if (c->q_heads % c->kv_heads != 0)
        return fail(KVC_ERR_SHAPE, "%s: q_heads %d is not a multiple of kv_heads %d", what,
                    c->q_heads, c->kv_heads);
    if (c->q_heads / c->kv_heads > 8)
        return fail(KVC_ERR_UNSUPPORTED, "%s: group size %d > 8", what, c->q_heads / c->kv_heads);
    if (c->head_dim != 128)
        return fail(KVC_ERR_UNSUPPORTED, "%s: head_dim %d (built: 128)", what, c->head_dim);
    if (c->bits != 4) return fail(KVC_ERR_UNSUPPORTED, "%s: bits %d (built: 4)", what, c->bits);
    if ((int64_t)c->batch * c->kv_heads > kMaxUnits)
        return fail(KVC_ERR_UNSUPPORTED, "%s: batch x kv_heads = %lld units > %d", what,
                    (long long)c->batch * c->kv_heads, kMaxUnits);
    if (c->max_quant % kvc::kKivGroup != 0)
        return fail(KVC_ERR_SHAPE, "%s: max_quant %d is not a multiple of %d", what, c->max_quant,
                    kvc::kKivGroup);
    if (!c->k_codes || !c->v_codes || !c->k_scale || !c->k_lo || !c->v_scale || !c->v_lo ||
        !c->k_res || !c->v_res || !c->n_quant || !c->n_res)
        return fail(KVC_ERR_INVALID_ARG, "%s: cache buffers must not be NULL", what);
    const void *al[] = {c->k_codes, c->v_codes, c->k_scale, c->k_lo, c->v_scale,
                        c->v_lo,    c->k_res,   c->v_res};
    for (const void *p : al)
        if ((uintptr_t)p % 16)
            return fail(KVC_ERR_INVALID_ARG, "%s: cache buffers must be 16-byte aligned", what);
    return KVC_OK;
}

// splits of the quantized tokens: shares of at most 128 groups (4,096
// tokens; each wave walks its own groups, so a long share costs no LDS, and
// one share per unit makes the step a single launch), enough splits for
// about 4,096 workgroups, no share under 4 groups, at most 64 splits; the
// last share of a unit also attends the residual and the new token, so there
// is always one
int kivi_nsq(const kvc_kivi_cache *c, int hint) {
    const int mq = (hint <= 0 || hint > c->max_quant) ? c->max_quant : hint;
    const int groups = mq / kvc::kKivGroup;
    if (groups == 0) return 1;
constexpr int kKivSplitGroups = 128;   // quantized groups per workgroup of the KIVI attention
    const int units = c->batch * c->kv_heads;
    int ns = (groups + kKivSplitGroups - 1) / kKivSplitGroups;
    const int fill = (4096 + units - 1) / units, by_len = (groups + 3) / 4;
    const int want = fill < by_len ? fill : by_len;
    ns = ns > want ? ns : want;
    return ns > 64 ? 64 : (ns < 1 ? 1 : ns);
}

// the shares' partials (read by the combine when a unit has several shares)
struct KiviWs {
    size_t part_q, total;
    int nsq;
};

KiviWs kivi_layout(const kvc_kivi_cache *c, int hint) {
    KiviWs w;
    const size_t units = (size_t)c->batch * c->kv_heads;
    const size_t G = (size_t)(c->q_heads / c->kv_heads);
    w.nsq = kivi_nsq(c, hint);
    const size_t pq = units * (size_t)w.nsq * G * (c->head_dim + 2) * sizeof(float);
    w.part_q = 0;
    w.total = align_up(pq);
    return w;
}

kvc::KiviArgs kivi_args(const kvc_kivi_cache *c) {
    kvc::KiviArgs a;
    memset(&a, 0, sizeof a);
    a.B = c->batch;
    a.Hq = c->q_heads;
    a.Hkv = c->kv_heads;
    a.G = c->q_heads / c->kv_heads;
    a.max_quant = c->max_quant;
    a.k_codes = c->k_codes;
    a.v_codes = c->v_codes;
    a.k_scale = c->k_scale;
    a.k_lo = c->k_lo;
    a.v_scale = c->v_scale;
    a.v_lo = c->v_lo;
    a.k_res = (uint16_t *)c->k_res;
    a.v_res = (uint16_t *)c->v_res;
    a.n_quant = c->n_quant;
    a.n_res = c->n_res;
    a.flags = c->flags;
    return a;
}

}  // namespace

KVC_EXPORT size_t kvc_kivi_workspace_bytes(const kvc_kivi_cache *c, int32_t max_quant_hint) {
    if (check_kivi(c, "kvc_kivi_workspace_bytes") != KVC_OK) return 0;
    return kivi_layout(c, max_quant_hint).total;
}

KVC_EXPORT kvc_status kvc_kivi_prefill(const kvc_kivi_cache *c, const void *k, const void *v,
                                       int32_t max_len, const int32_t *lengths, void *stream) {
    const char *what = "kvc_kivi_prefill";
    kvc_status s = check_kivi(c, what);
    if (s != KVC_OK) return s;
    if (max_len < 0) return fail(KVC_ERR_INVALID_ARG, "%s: max_len < 0", what);
    if (!lengths || (max_len > 0 && (!k || !v)))
        return fail(KVC_ERR_INVALID_ARG, "%s: k, v and lengths must not be NULL", what);
    if ((uintptr_t)k % 16 || (uintptr_t)v % 16)
        return fail(KVC_ERR_INVALID_ARG, "%s: k and v must be 16-byte aligned", what);
    const int over = max_len > kvc::kKivResidual ? max_len - kvc::kKivResidual : 0;
    const int64_t need = (int64_t)(over + kvc::kKivGroup - 1) / kvc::kKivGroup * kvc::kKivGroup;
    if (need > c->max_quant)
        return fail(KVC_ERR_SHAPE, "%s: %d prompt tokens need %lld quantized slots > max_quant %d",
                    what, max_len, (long long)need, c->max_quant);
    kvc::KiviArgs a = kivi_args(c);
    a.pk = (const uint16_t *)k;
    a.pv = (const uint16_t *)v;
    a.lengths = lengths;
    a.max_len = max_len;
    return hip_status(kvc::launch_kivi_prefill(a, (hipStream_t)stream), what);
}

KVC_EXPORT kvc_status kvc_kivi_decode(const kvc_kivi_cache *c, const void *q, const void *k_new,
                                      const void *v_new, float *out, float scale,
                                      int32_t max_quant_hint, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    const char *what = "kvc_kivi_decode";
    kvc_status s = check_kivi(c, what);
    if (s != KVC_OK) return s;
    if (!q || !k_new || !v_new || !out)
        return fail(KVC_ERR_INVALID_ARG, "%s: q, k_new, v_new and out must not be NULL", what);
    if ((uintptr_t)q % 16 || (uintptr_t)k_new % 16 || (uintptr_t)v_new % 16)
        return fail(KVC_ERR_INVALID_ARG, "%s: q, k_new and v_new must be 16-byte aligned", what);
    if (!isfinite(scale)) return fail(KVC_ERR_INVALID_ARG, "%s: scale is not finite", what);
    const KiviWs w = kivi_layout(c, max_quant_hint);
    if (!workspace)
        return fail(KVC_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", what, w.total);
    if (workspace_bytes < w.total)
        return fail(KVC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what,
                    workspace_bytes, w.total);
    if ((uintptr_t)workspace % kAlign)
        return fail(KVC_ERR_WORKSPACE, "%s: workspace must be %zu-byte aligned", what, kAlign);
    kvc::KiviArgs a = kivi_args(c);
    a.q = (const uint16_t *)q;
    a.k_new = (const uint16_t *)k_new;
    a.v_new = (const uint16_t *)v_new;
    a.out = out;
    a.scale = scale;
    a.nsq = w.nsq;
    a.part_q = (float *)((char *)workspace + w.part_q);
    return hip_status(kvc::launch_kivi_decode(a, (hipStream_t)stream), what);
}
