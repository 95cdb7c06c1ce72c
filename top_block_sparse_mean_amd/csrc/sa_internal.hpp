// sa_internal.hpp -- host-side launchers shared between the C ABI and the kernels.
#pragma once

#include "sa_common.hpp"

namespace sa {

enum { kSelectEmpty = 0, kSelectRow = 1, kSelectSplit = 2, kSelectTile = 3, kSelectHeads = 4, kSelectRowFused = 5 };

hipError_t launch_compress(const KP &P, int dtype, const void *k, float *k_cmp, int n_tail, hipStream_t st);
hipError_t launch_append(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                         float *k_cmp, hipStream_t st);

// The LSA flat bucket index: C tokens per cluster block, NB buckets per block, at most
// cap tokens per bucket, nblk blocks per (sequence, KV head) in the arrays.
struct BucketArgs {
    int C, NB, cap, nblk, from;
    float *centroid;      // [h_kv, batch, nblk, NB, d]
    int32_t *member;      // [h_kv, batch, nblk, C/g]
    int32_t *offset;      // [h_kv, batch, nblk, NB + 1]
};
hipError_t launch_bucket_build(const KP &P, const float *k_cmp, const BucketArgs &B, hipStream_t st);
size_t bucket_select_workspace_bytes(const KP &P, const BucketArgs &B, int kb);
hipError_t launch_bucket_select(const KP &P, int dtype, const void *q_sel, const BucketArgs &B, int kb, int32_t *idx,
                                int32_t *n_idx, void *ws, hipStream_t st);

// A decode step's append run by the selection kernel's launch (select.hip): the
// step's new keys and values, the cache they go to, the pooled keys to re-pool, and
// the blocks per sequence the pooling items cover (0: no append in the launch).
struct SelAppend {
    const void *k_new, *v_new;
    void *k, *v;
    float *k_cmp;
    int n_blk;
};
hipError_t launch_append_select(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                                float *k_cmp, const void *q_sel, int32_t *idx, int32_t *n_idx, void *ws,
                                hipStream_t st, void *ev0 = nullptr, void *ev1 = nullptr);

int select_plan(const KP &P);
size_t select_workspace_bytes(const KP &P, int plan);
hipError_t launch_select(const KP &P, int dtype, const void *q_sel, const float *k_cmp, const void *k,
                         int32_t *idx, int32_t *n_idx, void *ws, hipStream_t st, void *ev0 = nullptr,
                         void *ev1 = nullptr);

bool wg_fwd_ok(const KP &P, int dtype);
hipError_t launch_fwd_wg(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                         const int32_t *n_idx, void *out, float *lse, void *ev0, void *ev1, hipStream_t st);
bool tile_fwd_ok(const KP &P, int dtype);
hipError_t launch_fwd_tile(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                           const int32_t *n_idx, void *out, float *lse, void *ev0, void *ev1, hipStream_t st);
bool mfma_fwd_ok(const KP &P, int dtype);
int mfma_fwd_splits(const KP &P);
hipError_t launch_fwd_mfma(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                           const int32_t *n_idx, void *out, float *lse, void *ws, int splits, void *ev0, void *ev1,
                           hipStream_t st);

int fwd_splits(const KP &P);
size_t fwd_workspace_bytes(const KP &P, int splits);
hipError_t launch_fwd(const KP &P, int dtype, const void *q, const void *k, const void *v, const int32_t *idx,
                      const int32_t *n_idx, void *out, float *lse, void *ws, int splits, void *ev_begin,
                      void *ev_end, hipStream_t st);

// A decode step (append, select, attend) in one launch where it fits, else the three.
bool decode_step_fused_ok(const KP &P, int dtype, bool have_k_cmp);
hipError_t launch_decode_step(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                              float *k_cmp, const void *q, int32_t *idx, int32_t *n_idx, void *out, float *lse,
                              void *ws, int fwd_splits_n, hipStream_t st, void *ev0, void *ev1);

// Fixed device scratch of sparse_attn_fwd_noalloc (one array per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void **ptr);

// Contract checks: whether this build carries them, and the current device's
// check word (hipErrorNotSupported in a build without them).
bool contract_checked();
hipError_t contract_word(uint32_t **ptr);

} // namespace sa
