// abi.cpp -- the C ABI declared in include/sparse_attn.h: host-side validation,
// workspace sizing, status strings and dispatch to the kernel launchers.
// No device memory is allocated here; nothing is launched before every host
// check has passed.
#include "sparse_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "sa_internal.hpp"

namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

sa_status fail(sa_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

sa_status ok()
{
    g_last_error.clear();
    return SA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

sa_status check_params(const sa_params *p)
{
    if (!p)
        return fail(SA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1)
        return fail(SA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
    if (p->h_q < 1 || p->h_kv < 1 || p->h_q % p->h_kv != 0)
        return fail(SA_ERR_INVALID_ARG, "h_q (%d) must be a positive multiple of h_kv (%d)", p->h_q, p->h_kv);
    if (p->h_q / p->h_kv > 64)
        return fail(SA_ERR_UNSUPPORTED, "group size h_q/h_kv = %d exceeds 64", p->h_q / p->h_kv);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
    if (p->max_q < 1 || p->max_k < 1)
        return fail(SA_ERR_INVALID_ARG, "max_q (%d) and max_k (%d) must be >= 1", p->max_q, p->max_k);
    if (p->total_q < 1 || p->total_k < 1)
        return fail(SA_ERR_INVALID_ARG, "total_q (%lld) and total_k (%lld) must be >= 1", (long long)p->total_q,
                    (long long)p->total_k);
    if (p->total_q > (1LL << 40) || p->total_k > (1LL << 40) || p->max_k > (1 << 30))
        return fail(SA_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if ((long long)p->batch * p->h_kv > 65535 || (p->max_q + 63) / 64 > 65535)
        return fail(SA_ERR_UNSUPPORTED, "batch * h_kv must be <= 65535 and max_q <= 4194240");
    if (!p->cu_seqlens_q || !p->cu_seqlens_k)
        return fail(SA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k are required");
    if (p->block < 1)
        return fail(SA_ERR_INVALID_ARG, "block must be >= 1 (got %d)", p->block);
    if (p->pool != SA_POOL_MEAN && p->pool != SA_POOL_L2SUM)
        return fail(SA_ERR_INVALID_ARG, "unknown pool mode %d", p->pool);
    if (p->topk < 0)
        return fail(SA_ERR_INVALID_ARG, "topk must be >= 0 (got %d)", p->topk);
    if (p->topk > (1 << 24))                       // kernels index a row group's entries in 32 bits
        return fail(SA_ERR_UNSUPPORTED, "topk above 2^24 is not supported (got %d)", p->topk);
    if (p->n_init < 0)
        return fail(SA_ERR_INVALID_ARG, "n_init must be >= 0 (got %d)", p->n_init);
    if (p->window < 1)
        return fail(SA_ERR_INVALID_ARG, "window must be >= 1 (got %d): the attended set would be empty",
                    p->window);
    if (p->shared_selection != 0 && p->shared_selection != 1)
        return fail(SA_ERR_INVALID_ARG, "shared_selection must be 0 or 1");
    if (p->dtype != SA_DTYPE_F32 && p->dtype != SA_DTYPE_BF16)
        return fail(SA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    if (!(p->softmax_scale >= 0.f) || std::isinf(p->softmax_scale))
        return fail(SA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    if (p->pool_overlap < 0 || p->pool_overlap > (1 << 20))
        return fail(SA_ERR_INVALID_ARG, "pool_overlap must be in [0, 2^20] (got %d)", p->pool_overlap);
    if (p->select_mode != SA_SELECT_SUM && p->select_mode != SA_SELECT_SOFTMAX && p->select_mode != SA_SELECT_MAX &&
        p->select_mode != SA_SELECT_ATTN)
        return fail(SA_ERR_INVALID_ARG, "unknown select_mode %d", p->select_mode);
    if (p->select_mode == SA_SELECT_ATTN && (long long)(p->shared_selection ? p->max_q : 1) * (p->h_q / p->h_kv) > 64)
        return fail(SA_ERR_UNSUPPORTED, "SA_SELECT_ATTN: a row's queries times the group size must be <= 64");
    if (!(p->select_temperature >= 0.f) || std::isinf(p->select_temperature))
        return fail(SA_ERR_INVALID_ARG, "select_temperature must be finite and >= 0");
    if (p->block_table) {
        const int ps = p->page_size;
        if (ps < 1 || ps > (1 << 20) || (ps & (ps - 1)) != 0)
            return fail(SA_ERR_INVALID_ARG, "page_size must be a power of two in [1, 2^20] (got %d)", ps);
        const long long need = ((long long)p->max_k + ps - 1) / ps;
        if (p->max_pages < need)
            return fail(SA_ERR_INVALID_ARG, "max_pages (%d) below ceil(max_k / page_size) = %lld", p->max_pages,
                        need);
    }
    return SA_OK;
}

sa::KP make_kp(const sa_params *p)
{
    sa::KP k;
    k.batch = p->batch;
    k.h_q = p->h_q;
    k.h_kv = p->h_kv;
    k.d = p->head_dim;
    k.G = p->h_q / p->h_kv;
    k.max_q = p->max_q;
    k.max_k = p->max_k;
    k.total_q = p->total_q;
    k.total_k = p->total_k;
    k.cu_q = p->cu_seqlens_q;
    k.cu_k = p->cu_seqlens_k;
    k.q_pos0 = p->q_pos0;
    k.g = p->block;
    k.pool = p->pool;
    k.topk = p->topk;
    k.topk_per_seq = p->topk_per_seq;
    k.n_init = p->n_init;
    k.window = p->window;
    k.shared = p->shared_selection;
    k.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
    k.scale_log2 = k.scale * 1.4426950408889634f;
    k.nb_max = (p->max_k + p->block - 1) / p->block;
    k.rows = p->shared_selection ? p->batch : p->total_q;
    k.dtype = p->dtype;
    k.pool_overlap = p->pool_overlap;
    k.select_mode = p->select_mode;
    // per-head score scale: 1/tau for the softmax sum, 1/sqrt(d) otherwise
    k.head_score_scale = p->select_mode == SA_SELECT_SOFTMAX && p->select_temperature > 0.f
                             ? 1.0f / p->select_temperature
                             : 1.0f / std::sqrt((float)p->head_dim);
    k.attn_lse = p->attn_lse;
    k.bucket_c = k.bucket_nb = k.bucket_nblk = 0;
    k.boundary = nullptr;
    k.check = nullptr;
    if (sa::contract_checked()) {
        uint32_t *w = nullptr;
        if (sa::contract_word(&w) == hipSuccess)
            k.check = w;
    }
    // boundary scores in the select mode's units: the default mode ranks by the unscaled dot
    k.boundary_scale = p->select_mode == SA_SELECT_SUM ? 1.0f / std::sqrt((float)p->head_dim) : 1.0f;
    k.block_table = p->block_table;
    k.max_pages = p->block_table ? p->max_pages : 0;
    k.page_shift = 0;
    if (p->block_table)
        while ((1 << k.page_shift) < p->page_size)
            k.page_shift++;
    return k;
}

sa_status device_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return ok();
    return fail(SA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

} // namespace

extern "C" {

int sparse_attn_abi_version(void) { return SPARSE_ATTN_ABI_VERSION; }

const char *sparse_attn_status_string(int status)
{
    switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_DEVICE: return "HIP device error";
    }
    return "unknown status";
}

const char *sparse_attn_last_error(void) { return g_last_error.c_str(); }

sa_status sparse_attn_validate(const sa_params *p)
{
    sa_status s = check_params(p);
    return s == SA_OK ? ok() : s;
}

sa_status sparse_attn_workspace_size(const sa_params *p, size_t *select_bytes, size_t *fwd_bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    sa::KP k = make_kp(p);
    if (select_bytes)
        *select_bytes = sa::select_workspace_bytes(k, sa::select_plan(k));
    if (fwd_bytes)
        *fwd_bytes = sa::fwd_workspace_bytes(k, sa::fwd_splits(k));
    return ok();
}

static sa_status compress_common(const sa_params *p, int n_tail, const void *k, float *k_cmp, void *stream)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if (!k || !k_cmp)
        return fail(SA_ERR_INVALID_ARG, "k and k_cmp are required");
    if (!aligned16(k) || !aligned16(k_cmp))
        return fail(SA_ERR_INVALID_ARG, "k and k_cmp must be 16-byte aligned");
    sa::KP kp = make_kp(p);
    return device_status(sa::launch_compress(kp, p->dtype, k, k_cmp, n_tail, (hipStream_t)stream),
                         "compress launch");
}

sa_status sparse_attn_compress(const sa_params *p, const void *k, float *k_cmp, void *stream)
{
    return compress_common(p, 0, k, k_cmp, stream);
}

sa_status sparse_attn_compress_tail(const sa_params *p, int32_t n_tail_blocks, const void *k, float *k_cmp,
                                    void *stream)
{
    if (n_tail_blocks < 1)
        return fail(SA_ERR_INVALID_ARG, "n_tail_blocks must be >= 1 (got %d)", n_tail_blocks);
    return compress_common(p, n_tail_blocks, k, k_cmp, stream);
}

sa_status sparse_attn_append_kv(const sa_params *p, const void *k_new, const void *v_new, void *k, void *v,
                                float *k_cmp, void *stream)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if (!k_new || !v_new || !k || !v)
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k and v are required");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(v) || (k_cmp && !aligned16(k_cmp)))
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k, v and k_cmp must be 16-byte aligned");
    sa::KP kp = make_kp(p);
    return device_status(sa::launch_append(kp, p->dtype, k_new, v_new, k, v, k_cmp, (hipStream_t)stream),
                         "append launch");
}

static sa_status check_buckets(const sa_params *p, const sa_bucket_index *bx, sa::BucketArgs *out)
{
    if (!bx)
        return fail(SA_ERR_INVALID_ARG, "bucket index is NULL");
    const int g = p->block;
    if (bx->block_tokens < g || bx->block_tokens % g || bx->cap_tokens < g || bx->cap_tokens % g)
        return fail(SA_ERR_INVALID_ARG, "block_tokens (%d) and cap_tokens (%d) must be positive multiples of block",
                    bx->block_tokens, bx->cap_tokens);
    const int M = bx->block_tokens / g;
    if (M > 128)
        return fail(SA_ERR_UNSUPPORTED, "block_tokens / block = %d groups per cluster block exceeds 128", M);
    if (bx->count < 1 || bx->count > M)
        return fail(SA_ERR_INVALID_ARG, "count (%d) must be in [1, block_tokens / block = %d]", bx->count, M);
    if ((long long)(bx->cap_tokens / g) * bx->count < 2LL * M)
        return fail(SA_ERR_INVALID_ARG, "(cap_tokens / block) * count must be >= 2 * block_tokens / block");
    if (bx->blocks_max < p->max_k / bx->block_tokens || bx->blocks_max < 0)
        return fail(SA_ERR_INVALID_ARG, "blocks_max (%d) below max_k / block_tokens (%d)", bx->blocks_max,
                    p->max_k / bx->block_tokens);
    if (!bx->centroid || !bx->member || !bx->offset || !aligned16(bx->centroid))
        return fail(SA_ERR_INVALID_ARG, "centroid (16-byte aligned), member and offset are required");
    out->C = bx->block_tokens;
    out->NB = bx->count;
    out->cap = bx->cap_tokens;
    out->nblk = bx->blocks_max;
    if (bx->build_from < 0)
        return fail(SA_ERR_INVALID_ARG, "build_from must be >= 0 (got %d)", bx->build_from);
    out->from = bx->build_from;
    out->centroid = bx->centroid;
    out->member = bx->member;
    out->offset = bx->offset;
    return SA_OK;
}

sa_status sparse_attn_bucket_build(const sa_params *p, const float *k_cmp, const sa_bucket_index *bx, void *stream)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    sa::BucketArgs B;
    if ((s = check_buckets(p, bx, &B)) != SA_OK)
        return s;
    if (!k_cmp || !aligned16(k_cmp))
        return fail(SA_ERR_INVALID_ARG, "k_cmp is required (16-byte aligned)");
    sa::KP kp = make_kp(p);
    return device_status(sa::launch_bucket_build(kp, k_cmp, B, (hipStream_t)stream), "bucket build launch");
}

static sa_status check_bucket_select(const sa_params *p, const sa_bucket_index *bx, int32_t n_buckets,
                                     sa::BucketArgs *B)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if ((s = check_buckets(p, bx, B)) != SA_OK)
        return s;
    if (n_buckets < 1 || n_buckets > 1024)
        return fail(SA_ERR_INVALID_ARG, "n_buckets must be in [1, 1024] (got %d)", n_buckets);
    const long long need = (long long)n_buckets * (bx->cap_tokens / p->block);
    if (p->topk < need)
        return fail(SA_ERR_INVALID_ARG, "topk (%d, the table width) below n_buckets * cap_tokens / block = %lld",
                    p->topk, need);
    if (p->topk > 4096)
        return fail(SA_ERR_UNSUPPORTED, "bucket selection tables are at most 4096 groups wide (topk %d)", p->topk);
    return SA_OK;
}

sa_status sparse_attn_bucket_workspace_size(const sa_params *p, const sa_bucket_index *bx, int32_t n_buckets,
                                            size_t *bytes)
{
    sa::BucketArgs B;
    sa_status s = check_bucket_select(p, bx, n_buckets, &B);
    if (s != SA_OK)
        return s;
    if (bytes)
        *bytes = sa::bucket_select_workspace_bytes(make_kp(p), B, n_buckets);
    return ok();
}

sa_status sparse_attn_bucket_select(const sa_params *p, const void *q_sel, const sa_bucket_index *bx,
                                    int32_t n_buckets, int32_t *idx, int32_t *n_idx, void *ws, size_t ws_bytes,
                                    void *stream)
{
    sa::BucketArgs B;
    sa_status s = check_bucket_select(p, bx, n_buckets, &B);
    if (s != SA_OK)
        return s;
    if (!q_sel || !idx || !n_idx || !aligned16(q_sel))
        return fail(SA_ERR_INVALID_ARG, "q_sel (16-byte aligned), idx and n_idx are required");
    sa::KP kp = make_kp(p);
    const size_t need = sa::bucket_select_workspace_bytes(kp, B, n_buckets);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(SA_ERR_WORKSPACE, "bucket select needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    return device_status(sa::launch_bucket_select(kp, p->dtype, q_sel, B, n_buckets, idx, n_idx, ws,
                                                  (hipStream_t)stream),
                         "bucket select launch");
}

// The selection's arguments and workspace (after check_params).
static sa_status check_select(const sa_params *p, const void *q_sel, const float *k_cmp, const void *k,
                              const int32_t *idx, const int32_t *n_idx, const void *ws, size_t ws_bytes)
{
    if (!q_sel || !n_idx || (!idx && p->topk > 0))
        return fail(SA_ERR_INVALID_ARG, "q_sel, idx and n_idx are required");
    const bool attn = p->select_mode == SA_SELECT_ATTN;
    if ((p->block == 1 || attn) && !k)
        return fail(SA_ERR_INVALID_ARG, "block == 1 or SA_SELECT_ATTN scores the raw keys: k is required");
    if (p->block > 1 && !attn && !k_cmp)
        return fail(SA_ERR_INVALID_ARG, "block > 1 scores pooled keys: k_cmp is required");
    if (attn && !p->attn_lse)
        return fail(SA_ERR_INVALID_ARG, "SA_SELECT_ATTN needs attn_lse");
    if (!aligned16(q_sel) || (k && !aligned16(k)) || (k_cmp && !aligned16(k_cmp)))
        return fail(SA_ERR_INVALID_ARG, "q_sel, k and k_cmp must be 16-byte aligned");
    sa::KP kp = make_kp(p);
    int plan = sa::select_plan(kp);
    size_t need = sa::select_workspace_bytes(kp, plan);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SA_ERR_WORKSPACE, "select needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    return SA_OK;
}

sa_status sparse_attn_select(const sa_params *p, const void *q_sel, const float *k_cmp, const void *k,
                             int32_t *idx, int32_t *n_idx, float *boundary_scores, void *ws, size_t ws_bytes,
                             void *stream)
{
    sa_status s = check_params(p);
    if (s == SA_OK)
        s = check_select(p, q_sel, k_cmp, k, idx, n_idx, ws, ws_bytes);
    if (s != SA_OK)
        return s;
    if (boundary_scores && ((uintptr_t)boundary_scores & 3u))
        return fail(SA_ERR_INVALID_ARG, "boundary_scores must be 4-byte aligned");
    sa::KP kp = make_kp(p);
    kp.boundary = boundary_scores;
    return device_status(sa::launch_select(kp, p->dtype, q_sel, k_cmp, k, idx, n_idx, ws, (hipStream_t)stream,
                                           p->timing_events[0], p->timing_events[1]),
                         "select launch");
}

sa_status sparse_attn_append_select(const sa_params *p, const void *k_new, const void *v_new, void *k, void *v,
                                    float *k_cmp, const void *q_sel, int32_t *idx, int32_t *n_idx, void *ws,
                                    size_t ws_bytes, void *stream)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if (!k_new || !v_new || !k || !v)
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k and v are required");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(v) || (k_cmp && !aligned16(k_cmp)))
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k, v and k_cmp must be 16-byte aligned");
    if (p->select_mode == SA_SELECT_ATTN)
        return fail(SA_ERR_INVALID_ARG, "SA_SELECT_ATTN selects from a verify pass: use sparse_attn_select");
    s = check_select(p, q_sel, k_cmp, k, idx, n_idx, ws, ws_bytes);
    if (s != SA_OK)
        return s;
    sa::KP kp = make_kp(p);
    return device_status(sa::launch_append_select(kp, p->dtype, k_new, v_new, k, v, k_cmp, q_sel, idx, n_idx, ws,
                                                  (hipStream_t)stream, p->timing_events[0], p->timing_events[1]),
                         "append_select launch");
}

static sa_status check_fwd(const sa_params *p, const void *q, const void *k, const void *v, const int32_t *idx,
                           const int32_t *n_idx, const void *out)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if (!q || !k || !v || !out || !n_idx || (!idx && p->topk > 0))
        return fail(SA_ERR_INVALID_ARG, "q, k, v, out, idx and n_idx are required");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    return SA_OK;
}

sa_status sparse_attn_fwd(const sa_params *p, const void *q, const void *k, const void *v, const int32_t *idx,
                          const int32_t *n_idx, void *out, float *lse, void *ws, size_t ws_bytes, void *stream)
{
    sa_status s = check_fwd(p, q, k, v, idx, n_idx, out);
    if (s != SA_OK)
        return s;
    sa::KP kp = make_kp(p);
    int splits = sa::fwd_splits(kp);
    size_t need = sa::fwd_workspace_bytes(kp, splits);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SA_ERR_WORKSPACE, "fwd needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    return device_status(sa::launch_fwd(kp, p->dtype, q, k, v, idx, n_idx, out, lse, ws, splits,
                                        p->timing_events[0], p->timing_events[1], (hipStream_t)stream),
                         "fwd launch");
}

sa_status sparse_attn_decode_step(const sa_params *p, const void *k_new, const void *v_new, void *k, void *v,
                                  float *k_cmp, const void *q, int32_t *idx, int32_t *n_idx, void *out, float *lse,
                                  void *ws, size_t ws_bytes, void *stream)
{
    sa_status s = check_params(p);
    if (s != SA_OK)
        return s;
    if (!k_new || !v_new || !k || !v || !q || !out || !n_idx || (!idx && p->topk > 0))
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k, v, q, out, idx and n_idx are required");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(v) || !aligned16(q) ||
        !aligned16(out) || (k_cmp && !aligned16(k_cmp)))
        return fail(SA_ERR_INVALID_ARG, "k_new, v_new, k, v, q, out and k_cmp must be 16-byte aligned");
    if (p->select_mode == SA_SELECT_ATTN)
        return fail(SA_ERR_INVALID_ARG, "SA_SELECT_ATTN selects from a verify pass: use sparse_attn_select");
    if (p->block > 1 && !k_cmp)
        return fail(SA_ERR_INVALID_ARG, "block > 1 scores pooled keys: k_cmp is required");
    sa::KP kp = make_kp(p);
    const int splits = sa::fwd_splits(kp);
    size_t need = 0;
    if (!sa::decode_step_fused_ok(kp, p->dtype, k_cmp != nullptr)) {
        const size_t sb = sa::select_workspace_bytes(kp, sa::select_plan(kp));
        const size_t fb = sa::fwd_workspace_bytes(kp, splits);
        need = sb > fb ? sb : fb;
    }
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SA_ERR_WORKSPACE, "decode_step needs %zu bytes of 16-byte aligned workspace (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    return device_status(sa::launch_decode_step(kp, p->dtype, k_new, v_new, k, v, k_cmp, q, idx, n_idx, out, lse,
                                                ws, splits, (hipStream_t)stream, p->timing_events[0],
                                                p->timing_events[1]),
                         "decode_step launch");
}

sa_status sparse_attn_fwd_noalloc(const sa_params *p, const void *q, const void *k, const void *v,
                                  const int32_t *idx, const int32_t *n_idx, void *out, float *lse, void *stream)
{
    sa_status s = check_fwd(p, q, k, v, idx, n_idx, out);
    if (s != SA_OK)
        return s;
    sa::KP kp = make_kp(p);
    int splits = sa::fwd_splits(kp);
    size_t need = sa::fwd_workspace_bytes(kp, splits);
    if (need > sa::kNoAllocScratchBytes)
        return fail(SA_ERR_WORKSPACE, "fwd_noalloc: these parameters need %zu bytes of split partials, above the "
                    "fixed %zu-byte device scratch; use sparse_attn_fwd with a workspace", need,
                    sa::kNoAllocScratchBytes);
    void *scratch = nullptr;
    if (need > 0) {
        hipError_t e = sa::noalloc_scratch(&scratch);
        if (e != hipSuccess)
            return device_status(e, "fwd_noalloc scratch lookup");
    }
    return device_status(sa::launch_fwd(kp, p->dtype, q, k, v, idx, n_idx, out, lse, scratch, splits,
                                        p->timing_events[0], p->timing_events[1], (hipStream_t)stream),
                         "fwd_noalloc launch");
}

static_assert(SA_CHECK_SEQ == sa::kCheckSeq && SA_CHECK_TABLE == sa::kCheckTable && SA_CHECK_PAGE == sa::kCheckPage &&
                  SA_CHECK_TOKEN == sa::kCheckToken,
              "contract-check bits of the header and the kernels");

sa_status sparse_attn_check_flags(uint32_t *flags, int clear)
{
    if (!flags)
        return fail(SA_ERR_INVALID_ARG, "check_flags: flags is NULL");
    *flags = 0u;
    if (!sa::contract_checked())
        return fail(SA_ERR_UNSUPPORTED, "check_flags: this library is built without contract checks");
    uint32_t *word = nullptr;
    hipError_t e = sa::contract_word(&word);
    if (e != hipSuccess)
        return device_status(e, "check_flags: check word lookup");
    uint32_t v = 0u;
    e = hipMemcpy(&v, word, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return device_status(e, "check_flags: read");
    if (clear) {
        const uint32_t zero = 0u;
        e = hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice);
        if (e != hipSuccess)
            return device_status(e, "check_flags: clear");
    }
    *flags = v;
    return ok();
}

} // extern "C"
