/*
 * sparse_attn.h -- C ABI of selector-driven top-k block-sparse attention on
 * AMD Instinct MI355X (gfx950).
 *
 * One pass of the method is three calls on one HIP stream:
 *
 *   sparse_attn_compress  pool the keys of every block of `block` consecutive
 *                         tokens, per KV head: the mean (the parameter-free
 *                         mean pooling InfLLM-V2 uses; SparDA summary, Method)
 *                         or the sum of L2-normalised keys (LSA deep-read, §2.2,
 *                         4 keys pooled into one).
 *   sparse_attn_select    score every candidate block with the query heads of a
 *                         GQA group summed into one selector query,
 *                         s_j = (sum_h q_h) . K~_j / sqrt(d) (SparDA summary,
 *                         Method: one selector head per GQA group; LSA
 *                         deep-read, §2.3-§2.4: one index table shared by all
 *                         heads), keep the top-k, ties to the lower index.
 *   sparse_attn_fwd       softmax attention restricted to the union of the init
 *                         (sink) tokens, the local window and the selected blocks
 *                         (PulseCol, §3.1 Eq. (1)-(2); S3R review, sparse drafting
 *                         formula; SparDA summary, Method), online softmax with
 *                         fp32 accumulation.
 *
 * Definitions used by every call (positions are 0-based, per sequence):
 *   query i of sequence b sits at p = q0_b + i, q0_b = q_pos0[b] or N_b - M_b;
 *   selection position p_sel = p (per-query selection), or q0_b - 1 for the one
 *     row of sequence b when shared_selection = 1 (S3R drafts: the history up
 *     to the verification boundary is selected once and reused by every draft);
 *   block j = tokens [j*g, min((j+1)*g, N_b) - 1] = [j*g, e_j];
 *   F(p_sel) = [0, min(n_init, p_sel+1)) U [max(0, p_sel-window+1), p_sel];
 *   candidates C = { j : e_j <= p_sel and block j is not wholly inside F };
 *   selected S = the first min(k, |C|) of C ordered by (score desc, j asc);
 *   attended set A(p) = { t <= p : t < n_init, or t >= p_sel-window+1, or t in
 *     a block of S }.
 *
 * Conventions:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates or frees device memory and keeps no state between calls.
 *   - Q/K/V/O and k_cmp must be 16-byte aligned; all are row-major with the
 *     head dimension contiguous.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Scalar and shape arguments are checked on the host before any HIP call;
 *     a failed check returns a status and enqueues nothing.  Device-resident
 *     contents (cu_seqlens monotone, q_pos0[b] + M_b <= N_b, topk_per_seq[b] <=
 *     topk, finite inputs) are the caller's contract and are not checked.
 *   - Nothing throws across the ABI.  sparse_attn_last_error() returns the
 *     detail of the calling thread's last failure.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_ABI_VERSION 10

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1, /* bad scalar, shape, pointer or alignment            */
    SA_ERR_UNSUPPORTED = 2, /* valid but not built (e.g. head_dim not 64 or 128)  */
    SA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required          */
    SA_ERR_DEVICE = 4       /* a HIP launch or runtime call failed                 */
} sa_status;

typedef enum sa_dtype { SA_DTYPE_F32 = 0, SA_DTYPE_BF16 = 1 } sa_dtype;
typedef enum sa_pool { SA_POOL_MEAN = 0, SA_POOL_L2SUM = 1 } sa_pool;

/* How the query heads of a GQA group combine into one block score. */
typedef enum sa_select_mode {
    SA_SELECT_SUM = 0,     /* (sum_h q_h) . K~_j / sqrt(d): the heads summed into one selector query */
    SA_SELECT_SOFTMAX = 1, /* sum_h softmax_j(q_h . K~_j / tau) over the row's candidates (SparDA
                              summary, Method: the target score of its indexer)                  */
    SA_SELECT_MAX = 2,     /* max_h q_h . K~_j / sqrt(d) (LSA deep-read, §2.5: a bucket scored by
                              its best head)                                                       */
    SA_SELECT_ATTN = 3     /* the attention mass a dense verify pass puts on block j: the sum over
                              the row's queries i, the group's heads h and the block's tokens t of
                              exp(scale q_ih . k_t - lse_ih), lse from that pass (S3R review: the
                              verifier's attention refreshes the next drafts' subset); reads the
                              raw keys                                                            */
} sa_select_mode;

typedef struct sa_params {
    int32_t batch;             /* B >= 1 sequences                                      */
    int32_t h_q, h_kv;         /* query / KV heads; h_q % h_kv == 0, G = h_q / h_kv <= 64 */
    int32_t head_dim;          /* d: 64 or 128                                          */
    int32_t max_q, max_k;      /* upper bounds on every M_b and N_b (grid sizing; the
                                  pooled-key rows nbmax = ceil(max_k / block) per
                                  sequence, so a decode loop keeps one k_cmp, sized
                                  for its capacity, as its sequences grow)           */
    int64_t total_q, total_k;  /* sum M_b and sum N_b: rows of Q/O and of K/V           */
    const int32_t *cu_seqlens_q; /* device [batch+1], packed query offsets, [0] = 0     */
    const int32_t *cu_seqlens_k; /* device [batch+1], packed key offsets, [0] = 0       */
    const int32_t *q_pos0;     /* device [batch] absolute position of query 0, or NULL  */
    int32_t block;             /* g >= 1 tokens per pooled block (g = 1: token level)   */
    int32_t pool;              /* sa_pool                                               */
    int32_t topk;              /* k in [0, 2^24] blocks per row; the row capacity of `idx`
                                  (larger: SA_ERR_UNSUPPORTED)                          */
    const int32_t *topk_per_seq; /* device [batch] per-sequence k (each <= topk), or NULL */
    int32_t n_init;            /* sink tokens >= 0                                      */
    int32_t window;            /* local window in tokens >= 1                           */
    int32_t shared_selection;  /* 0: one row per query; 1: one row per sequence         */
    float softmax_scale;       /* attention logit scale; 0 => 1/sqrt(head_dim)          */
    int32_t dtype;             /* sa_dtype of Q, K, V and O                             */
    void *timing_events[2];    /* optional hipEvent_t pair: when both are set,
                                  sparse_attn_fwd records [0] right before and [1]
                                  right after its main attention kernel on `stream`,
                                  sparse_attn_select around its scoring kernel (the
                                  one that reads the keys; the top-k follows)       */
    /* Paged K/V cache (optional; NULL block_table = the packed layout above).
     * With a block table every K and V argument of every call is a page pool
     * [pool_rows, h_kv, d] and token t of sequence b is pool row
     *   block_table[b * max_pages + t / page_size] * page_size + t % page_size;
     * cu_seqlens_k then only gives the lengths N_b, and total_k is still sum N_b.
     * The pool must hold fewer than 2^31 rows; page ids are the caller's
     * contract (not checked).  Pooled keys, Q/O and the selection table keep
     * their layouts. */
    const int32_t *block_table; /* device [batch, max_pages] int32 page ids, or NULL  */
    int32_t max_pages;         /* row stride of block_table; >= ceil(max_k / page_size) */
    int32_t page_size;         /* tokens per page: a power of two, 1 .. 2^20           */
    /* Selector variants (zero = the definitions above). */
    int32_t pool_overlap;      /* o >= 0: block j pools tokens [max(0, j*g - o), e_j], a window of
                                  g + o tokens at stride g (InfLLM-V2's overlapping compressed keys,
                                  SparDA summary, Method); block j is still tokens [j*g, e_j]      */
    int32_t select_mode;       /* sa_select_mode; with several queries in a row, q_h sums head h
                                  over them                                                       */
    float select_temperature;  /* tau of SA_SELECT_SOFTMAX; 0 => sqrt(head_dim)                    */
    const float *attn_lse;     /* SA_SELECT_ATTN: device [h_q, total_q] natural-log log-sum-exp of
                                  each (query, head) over every key up to its position, as
                                  sparse_attn_fwd writes it for a table that keeps every candidate;
                                  the row's queries times G must be <= 64                          */
} sa_params;

/* The LSA flat bucket index (LSA deep-read, §2.2-§2.3): every complete cluster block
 * of block_tokens consecutive tokens (block_tokens / block pooled groups of one
 * sequence and KV head) is clustered bottom-up by Ward's criterion into `count`
 * buckets of at most cap_tokens tokens; a bucket's centroid is the normalised sum of
 * its members' pooled keys.  The arrays are owned by the caller. */
typedef struct sa_bucket_index {
    int32_t block_tokens;      /* C: a multiple of block, with C / block <= 128              */
    int32_t count;             /* NB buckets per cluster block, 1 <= NB <= C / block          */
    int32_t cap_tokens;        /* a multiple of block; (cap_tokens / block) * NB >= 2 C / block
                                  (merging never stalls above NB buckets)                     */
    int32_t blocks_max;        /* cluster blocks per (sequence, KV head) in the arrays,
                                  >= max_k / C (only complete blocks hold buckets)            */
    float *centroid;           /* device [h_kv, batch, blocks_max, NB, d] fp32                */
    int32_t *member;           /* device [h_kv, batch, blocks_max, C / block]: each block's
                                  group indices, grouped by bucket (buckets ordered by their
                                  smallest member), ascending within a bucket; -1 for a block
                                  that is not complete                                         */
    int32_t *offset;           /* device [h_kv, batch, blocks_max, NB + 1]: bucket i holds
                                  member[offset[i] .. offset[i+1])                             */
    int32_t build_from;        /* sparse_attn_bucket_build leaves cluster blocks before this
                                  one untouched (a stream of chunks clusters each block once,
                                  as it completes; buckets are frozen once built)             */
} sa_bucket_index;

/* SPARSE_ATTN_ABI_VERSION of the built library. */
int sparse_attn_abi_version(void);

/* Static description of a status code (an sa_status value; any other value reads
 * "unknown status"); never NULL. */
const char *sparse_attn_status_string(int status);

/* Detail of the calling thread's last non-OK status ("" if none); never NULL. */
const char *sparse_attn_last_error(void);

/* Host-only check of every scalar and shape field; touches no device. */
sa_status sparse_attn_validate(const sa_params *p);

/* Bytes of device workspace that sparse_attn_select and sparse_attn_fwd need
 * for these parameters (either pointer may be NULL).  0 means none needed. */
sa_status sparse_attn_workspace_size(const sa_params *p, size_t *select_bytes, size_t *fwd_bytes);

/* Pool the keys (SparDA summary, Method: InfLLM-V2 mean pooling of keys; LSA
 * deep-read, §2.2: L2-normalise, then sum consecutive keys).
 *   k      [total_k, h_kv, d] of dtype
 *   k_cmp  [h_kv, batch, nbmax, d] fp32, nbmax = ceil(max_k / block); block j of
 *          sequence b holds the mean (SA_POOL_MEAN) or the sum of k/|k|_2
 *          (SA_POOL_L2SUM, a zero key adds zero) over the block's pooling
 *          window (its tokens and the pool_overlap tokens before them), the
 *          last block of a sequence over the tokens it has.  Rows
 *          j >= ceil(N_b / block) are not written. */
sa_status sparse_attn_compress(const sa_params *p, const void *k, float *k_cmp, void *stream);

/* Recompute only the last n_tail_blocks pooled blocks of every sequence (the
 * ones a decode step that appends keys changes); same layout and values as
 * sparse_attn_compress for those rows.  n_tail_blocks >= 1. */
sa_status sparse_attn_compress_tail(const sa_params *p, int32_t n_tail_blocks, const void *k,
                                    float *k_cmp, void *stream);

/* Append the newest keys and values of every sequence to its cache and re-pool
 * the blocks they fall in (the decode-time update of the pooled keys: a block
 * that is still filling is pooled over the tokens it has and pooled again as
 * tokens arrive, which keeps K~ equal to a fresh sparse_attn_compress of the
 * grown cache; SparDA summary, Method; LSA deep-read, §2.2).  The parameters
 * describe the cache AFTER the append: the M_b rows of sequence b in
 * cu_seqlens_q are its new tokens, at positions q0_b .. q0_b + M_b - 1
 * (q0_b = q_pos0[b] or N_b - M_b, as for queries).
 *   k_new, v_new  [total_q, h_kv, d] of dtype: the new keys and values
 *   k, v          the cache, packed [total_k, h_kv, d] or paged (block_table);
 *                 the new rows are written, no other row is
 *   k_cmp         pooled keys as from sparse_attn_compress; the blocks holding a
 *                 new token are recomputed from the cache, or NULL to skip
 *                 pooling (always skipped when block == 1)
 * One kernel on `stream`: with pooling, one workgroup per (sequence, KV head,
 * touched block) writes the new rows of that block and pools its window, taking
 * the new tokens from k_new and the others from the cache; without, a row
 * scatter. */
sa_status sparse_attn_append_kv(const sa_params *p, const void *k_new, const void *v_new, void *k, void *v,
                                float *k_cmp, void *stream);

/* Top-k block selection (SparDA summary, Method; LSA deep-read, §2.3; S3R
 * review, sparse drafting: recent window + top-K by score).
 *   q_sel  [total_q, h_q, d] of dtype: the selector queries (Q itself, or a
 *          separate selector projection of the same shape)
 *   k_cmp  pooled keys from sparse_attn_compress; ignored when block == 1 (the
 *          raw keys `k` are scored) or select_mode == SA_SELECT_ATTN, and may then
 *          be NULL
 *   k      [total_k, h_kv, d] (or the paged pool); read when block == 1 or
 *          select_mode == SA_SELECT_ATTN (else may be NULL)
 *   idx    [h_kv, rows, topk] int32 out: selected block indices of each row in
 *          ascending order, padded with -1; rows = total_q, or batch when
 *          shared_selection = 1
 *   n_idx  [h_kv, rows] int32 out: number of selected blocks, min(k, |C|)
 *   boundary_scores  [h_kv, rows, 2] fp32 out, or NULL: the row's need-th and
 *          (need+1)-th largest scores, need = min(k, |C|) (the smallest score
 *          kept and the largest left out), taken from the very fp32 values the
 *          selection ranked, in the select mode's units (the default mode's
 *          dot times 1/sqrt(d); the other modes' scores as they are); both NaN
 *          for a row that keeps every candidate or none (nothing is ranked).
 *          This is the near-tie audit of the stated tie rule: a row whose two
 *          values differ by < 1e-4 relative sits on a near tie.  Costs an extra
 *          pass over the scores on plans that keep them in the workspace.
 *   ws     workspace of at least select_bytes (sparse_attn_workspace_size),
 *          owned by the caller; its contents on entry do not matter.  Calls
 *          that share one workspace must not overlap in time.
 * Scores are computed in fp32 from fp32 pooled keys and fp32-summed queries;
 * equal scores keep the lower block index. */
sa_status sparse_attn_select(const sa_params *p, const void *q_sel, const float *k_cmp,
                             const void *k, int32_t *idx, int32_t *n_idx, float *boundary_scores,
                             void *ws, size_t ws_bytes, void *stream);

/* A decode step's append and selection in one call: the same results as
 * sparse_attn_append_kv(p, k_new, v_new, k, v, k_cmp) followed by
 * sparse_attn_select(p, q_sel, k_cmp, k, idx, n_idx, ws).  For decode rows (one
 * query per sequence, block > 1 with k_cmp, window >= block, a batch whose rows x
 * KV heads fill the GPU) one launch does both: the workgroup that selects for a
 * sequence and KV head first writes that sequence's new token and re-pools the
 * blocks whose pooling window holds it, none of which can be a candidate (the
 * token's own block lies inside the window).  Otherwise two launches.  Arguments as
 * for those two calls (select_mode SA_SELECT_ATTN is rejected: it selects from a
 * verify pass); ws of select_bytes. */
sa_status sparse_attn_append_select(const sa_params *p, const void *k_new, const void *v_new, void *k,
                                    void *v, float *k_cmp, const void *q_sel, int32_t *idx, int32_t *n_idx,
                                    void *ws, size_t ws_bytes, void *stream);

/* Build the bucket index from pooled keys (LSA deep-read, §2.2: streaming Ward
 * clustering into buckets, centroids = normalised member sums).  Every round, each
 * bucket finds its cheapest partner by Ward's criterion among the buckets it may join
 * (merged size within cap); pairs that are each other's cheapest merge -- the cheapest
 * pairs (by cost, then the lower bucket) when all would leave fewer than NB buckets --
 * until NB buckets remain.  Costs are fp32: |n_B S_A - n_A S_B|^2 / (n_A n_B (n_A + n_B))
 * with S the member sums and n the sizes, accumulated with fused multiply-adds over the
 * head dimension in order.  Blocks that are not complete are marked (member -1).
 *   k_cmp  pooled keys [h_kv, batch, nbmax, d] from sparse_attn_compress */
sa_status sparse_attn_bucket_build(const sa_params *p, const float *k_cmp, const sa_bucket_index *bx, void *stream);

/* Bytes of workspace sparse_attn_bucket_select needs for n_buckets per row. */
sa_status sparse_attn_bucket_workspace_size(const sa_params *p, const sa_bucket_index *bx, int32_t n_buckets,
                                            size_t *bytes);

/* Flat bucket retrieval (LSA deep-read, §2.3): the row's selector query (the group's
 * heads summed, as in sparse_attn_select) scores the centroids of the complete
 * cluster blocks that end at or before the row's selection position, the n_buckets
 * best (ties to the lower bucket) are taken and expanded to all their member groups.
 *   idx    [h_kv, rows, topk] out: the groups, ascending, -1 padded; topk (the table
 *          width, which sparse_attn_fwd reads too) must be >= n_buckets * cap_tokens /
 *          block and <= 4096
 *   n_idx  [h_kv, rows] out: the number of groups
 *   n_buckets in [1, 1024]; ws of sparse_attn_bucket_workspace_size bytes. */
sa_status sparse_attn_bucket_select(const sa_params *p, const void *q_sel, const sa_bucket_index *bx,
                                    int32_t n_buckets, int32_t *idx, int32_t *n_idx, void *ws, size_t ws_bytes,
                                    void *stream);

/* Sparse attention over A(p) for every query and query head (PulseCol, §3.1
 * Eq. (2); S3R review, sparse drafting formula).
 *   q      [total_q, h_q, d]; k, v [total_k, h_kv, d]; all of dtype
 *   idx, n_idx  a selection table as written by sparse_attn_select
 *   out    [total_q, h_q, d] of dtype
 *   lse    [h_q, total_q] fp32 natural-log sum of exp of the scaled logits, or NULL
 *   ws     workspace of at least fwd_bytes (sparse_attn_workspace_size).
 * Logits, the running max and sum and the output accumulator are fp32. */
sa_status sparse_attn_fwd(const sa_params *p, const void *q, const void *k, const void *v,
                          const int32_t *idx, const int32_t *n_idx, void *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream);

/* One decode step: the same results as sparse_attn_append_kv(p, k_new, v_new, k, v,
 * k_cmp), then sparse_attn_select(p, q, k_cmp, k, idx, n_idx, NULL, ...), then
 * sparse_attn_fwd(p, q, k, v, idx, n_idx, out, lse, ...) -- the selector query is the
 * attention query.  For bf16 decode rows (one query per sequence, block > 1 with k_cmp,
 * window >= block, the default group score, G <= 8, a batch whose rows x KV heads fill
 * the GPU, attended sets of at most 8192 tokens) one launch does all three: the
 * workgroup of a (sequence, KV head) appends, selects and then attends with its
 * selection kept in LDS (the selection equals the separate calls' bit for bit; the
 * output and lse agree with sparse_attn_fwd's to fp32 rounding of a different
 * summation order).  Otherwise the three calls run in turn.  idx and n_idx are
 * written either way.  ws: at least the larger of select_bytes and fwd_bytes
 * (sparse_attn_workspace_size), or none when the step runs in one launch.
 * timing_events bracket the one launch, or the attention kernel otherwise. */
sa_status sparse_attn_decode_step(const sa_params *p, const void *k_new, const void *v_new, void *k, void *v,
                                  float *k_cmp, const void *q, int32_t *idx, int32_t *n_idx, void *out,
                                  float *lse, void *ws, size_t ws_bytes, void *stream);

/* sparse_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the split partials kept in a fixed 32 MiB
 * device array that the library holds on each GPU it runs on until the process
 * ends, instead of a caller workspace.  Arguments as for sparse_attn_fwd less
 * the workspace.  Parameters whose partials would exceed 32 MiB (fwd_bytes of
 * sparse_attn_workspace_size) return SA_ERR_WORKSPACE before any HIP call.
 * The first call on a device looks up the array's address (no allocation).
 * Every call on one GPU shares that array, so calls that overlap in time on one
 * GPU (other streams, other threads) race; it needs no clearing (every split
 * writes all its partials before the combine reads them). */
sa_status sparse_attn_fwd_noalloc(const sa_params *p, const void *q, const void *k, const void *v,
                                  const int32_t *idx, const int32_t *n_idx, void *out, float *lse,
                                  void *stream);

/* Contract checks, a debugging aid (no passage of the pages defines it).  The
 * library built with contract checks (libsparse_attn_checked.so: every kernel
 * compiled with SA_CHECKED) validates what its kernels read through the caller's
 * device tables and, for each kind of violation it meets, sets one bit in a word
 * it keeps on each GPU; the access then takes a clamped index inside the caller's
 * buffers, so a call with broken tables returns wrong numbers, not a fault:
 *   SA_CHECK_SEQ    sequence geometry: cu_seqlens not non-decreasing, a length
 *                   above max_q / max_k or past total_q / total_k, q_pos0 + M_b > N_b
 *   SA_CHECK_TABLE  selection table: n_idx outside [0, topk], an entry outside its
 *                   row's candidate blocks, entries not ascending
 *   SA_CHECK_PAGE   block table: a negative page id (pages past the end of the
 *                   pool cannot be seen: the pool size is not passed)
 *   SA_CHECK_TOKEN  a gathered token outside [0, p] of its query
 * sparse_attn_check_flags copies the current GPU's word into *flags (host memory)
 * and zeroes it when clear != 0.  The copy is synchronous: call it once the
 * checked work is done (its streams synchronised).  In a build without checks it
 * sets *flags = 0 and returns SA_ERR_UNSUPPORTED; NULL flags gives
 * SA_ERR_INVALID_ARG, a failed HIP call SA_ERR_DEVICE.  Checked builds are for
 * tests and debugging: the checks cost time in every kernel that gathers. */
#define SA_CHECK_SEQ 1u
#define SA_CHECK_TABLE 2u
#define SA_CHECK_PAGE 4u
#define SA_CHECK_TOKEN 8u
sa_status sparse_attn_check_flags(uint32_t *flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
