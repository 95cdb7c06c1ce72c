// append_common.hpp -- the decode-time append as workgroup-sized work items, shared
// by the append kernels (compress.hip) and the decode selection kernel that runs the
// append in its own launch (select.hip).
//
// The append writes each sequence's newest keys and values to its cache rows and
// re-pools every block whose pooling window holds a new token (SparDA summary,
// Method: InfLLM-V2 pools keys by a parameter-free mean; LSA deep-read, §2.2: the
// sum of L2-normalised keys), so the pooled keys stay equal to a fresh pooling of
// the grown cache.
#pragma once

#include "sa_common.hpp"

namespace sa {

// Which pooled rows a launch computes: every block, the last n_blk_iter blocks of
// each sequence, or the blocks holding a sequence's query positions (the tokens an
// append wrote).  Returns false when jj is past the sequence's range.
enum { kPoolAll = 0, kPoolTail = 1, kPoolAppended = 2 };

__device__ __forceinline__ bool pooled_block(const KP &P, const Seq &s, int mode, int n_blk_iter, int jj, int &j)
{
    const int nb = (s.n_k + P.g - 1) / P.g;
    int last = nb - 1;
    if (mode == kPoolAll) {
        j = jj;
    } else if (mode == kPoolTail) {
        j = nb - n_blk_iter + jj;
    } else {
        j = s.q0 / P.g + jj;          // a token also lies in the windows of the blocks up to o tokens after it
        last = s.n_q > 0 ? min(last, (s.q0 + s.n_q - 1 + P.pool_overlap) / P.g) : -1;
    }
    return j >= 0 && j <= last && j < P.nb_max;
}

// Blocks per sequence an append may touch: M consecutive tokens lie in the pooling
// windows of at most ceil((M + o) / g) + 1 blocks.
__host__ __forceinline__ int append_pool_blocks(const KP &P)
{
    long long n_blk = ((long long)P.max_q + P.pool_overlap + P.g - 1) / P.g + 1;
    return (int)(n_blk < P.nb_max ? n_blk : P.nb_max);
}

// Copy of one token's 16-byte piece: k_new / v_new row i -> cache row `row`.
template <typename T>
__device__ __forceinline__ void copy_piece(const T *src, T *dst, long long src_row, long long dst_row, int width,
                                           int x)
{
    reinterpret_cast<uint4 *>(dst + dst_row * width)[x] = reinterpret_cast<const uint4 *>(src + src_row * width)[x];
}

// No pooling (g = 1 or no pooled keys), item i = new token row i: its h_kv x d keys
// and values go to the cache row of position q0_b + (i - q_off).  256 threads.
template <typename T>
__device__ __forceinline__ void append_rows_item(const KP &P, const T *k_new, const T *v_new, T *k, T *v,
                                                 long long i)
{
    const int b = seq_of_query(P, i);
    const Seq s = seq_info(P, b);
    const long long row = kv_base(P, s) + kv_map(P, b).row(s.q0 + (int)(i - s.q_off));
    const int width = P.h_kv * P.d, pieces = width * (int)sizeof(T) / 16;
    for (int x = threadIdx.x; x < pieces; x += 256) {
        copy_piece(k_new, k, i, row, width, x);
        copy_piece(v_new, v, i, row, width, x);
    }
}

// With pooling, item = (sequence, KV head, touched block) over append_pool_blocks
// blocks per sequence.  New tokens in the block's pooling window are taken from
// k_new / v_new (and written to the cache when they belong to the block itself);
// its other tokens are read from the cache; the window is pooled as the pooling
// kernels pool it.  Each new (token, head) belongs to one block, so every cache row
// is written by one item, and no item reads a row another writes.  The first 256
// threads do the work (the same summation order whatever the workgroup size); every
// thread of the workgroup calls it, and it ends with a barrier, so a workgroup may
// run several items in turn.  UN token rounds of the pooling window are loaded at a
// time (registers against memory latency; the sums run in token order whatever UN).
template <typename T, int D, int POOL, int UN = 4>
__device__ __forceinline__ void append_pool_item(const KP &P, const T *k_new, const T *v_new, T *k, T *v,
                                                 float *k_cmp, int n_blk_iter, long long item)
{
    constexpr int L = D / 8, TG = 256 / L;
    __shared__ float sh[TG][D];
    const int jj = (int)(item % n_blk_iter);
    const int c = (int)((item / n_blk_iter) % P.h_kv);
    const int b = (int)(item / ((long long)n_blk_iter * P.h_kv));
    const int tid = threadIdx.x, chunk = tid % L, tg = tid / L;
    const bool act = tid < 256;
    const Seq s = seq_info(P, b);
    const long long k_base = kv_base(P, s);
    const KvMap map = kv_map(P, b);
    int j;
    if (!pooled_block(P, s, kPoolAppended, n_blk_iter, jj, j))
        return;
    const int t0 = max(0, j * P.g - P.pool_overlap), t1 = min(j * P.g + P.g, s.n_k);   // pooling window
    // UN token rounds of the window are loaded before any is summed (with UN = 4 the
    // window of a 64-token block is one memory latency instead of four); the sums run
    // in token-round order as without the batching.
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it0 = 0; it0 < P.g + P.pool_overlap; it0 += UN * TG) {
        float x[UN][8];
#pragma unroll
        for (int u = 0; u < UN; u++) {
            const int t = t0 + it0 + u * TG + tg;
#pragma unroll
            for (int e = 0; e < 8; e++)
                x[u][e] = 0.f;
            if (act && t < t1) {
                const long long crow = (k_base + map.row(t)) * P.h_kv + c;
                if (t >= s.q0 && t < s.q0 + s.n_q) {
                    const long long nrow = (s.q_off + (t - s.q0)) * P.h_kv + c;
                    load8(k_new + nrow * D + chunk * 8, x[u]);
                    constexpr int PPC = 8 * (int)sizeof(T) / 16;        // 16-byte pieces per 8 elements
                    if (t >= j * P.g)                                    // the block's own tokens only
#pragma unroll
                        for (int w = 0; w < PPC; w++) {
                            copy_piece(k_new, k, nrow, crow, D, chunk * PPC + w);
                            copy_piece(v_new, v, nrow, crow, D, chunk * PPC + w);
                        }
                } else {
                    load8(k + crow * D + chunk * 8, x[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UN; u++) {
            float sc = 1.0f;
            if (POOL == 1) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    ss += x[u][e] * x[u][e];
                ss = group_sum<L>(ss);
                sc = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; e++)
                acc[e] += x[u][e] * sc;
        }
    }
    if (act)
#pragma unroll
        for (int e = 0; e < 8; e++)
            sh[tg][chunk * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
        for (int g2 = 0; g2 < TG; g2++)
            sum += sh[g2][tid];
        if (POOL == 0)
            sum *= 1.0f / (float)(t1 - t0);
        k_cmp[(((long long)c * P.batch + b) * P.nb_max + j) * D + tid] = sum;
    }
    __syncthreads();                  // sh is free again
}

// The append item of a one-token decode step (bf16) in three parts, so that its memory
// latency can hide behind other work of the same workgroup: append_split_issue loads
// the pooling window of the block that holds the sequence's new token (that token from
// k_new, the others from the cache) and the new token's value piece;
// append_split_commit, any time later, adds up each lane's tokens into LDS partials and
// writes the new token's key and value pieces to the cache; append_split_store, after a
// barrier, writes the pooled row.  The sums and their order are append_pool_item's.
// One round of loads: g + o <= UN * TG (append_split_fits).  For one new token per
// sequence (right-aligned, n_q = 1): the block of append item 0 is the only one it
// touches.
template <int D, int UN = 4>
struct AppendSplit {
    uint4 raw[UN];            // 8 bf16 keys per lane and token round (valid bit u: inside the window)
    uint32_t valid;
    int j, t0, t1;            // the pooled block, its pooling window [t0, t1)
    bool ok;                  // the block exists
};

template <int D, int UN = 4>
__host__ __device__ __forceinline__ bool append_split_fits(const KP &P)
{
    return P.g + P.pool_overlap <= UN * (256 / (D / 8));
}

// s, map: the sequence's geometry and cache map (seq_info, kv_map).  No load result
// is used here, so nothing waits for them.  knew / vnew: the new token's key and value
// pieces, crow_new its cache row (-1 in lanes that do not hold it), kept apart from the
// struct (inside it, the compiler staged them through memory, which waits for the load).
template <int D, int UN>
__device__ __forceinline__ void append_split_issue(const KP &P, const Seq &s, const KvMap &map,
                                                   const uint16_t *k_new, const uint16_t *v_new, const uint16_t *k,
                                                   int n_blk_iter, int c, AppendSplit<D, UN> &a, uint4 &knew,
                                                   uint4 &vnew, long long &crow_new)
{
    constexpr int L = D / 8, TG = 256 / L;
    const int tid = threadIdx.x, chunk = tid % L, tg = tid / L;
    const bool act = tid < 256;
    const long long k_base = kv_base(P, s);
    crow_new = -1;
    a.valid = 0u;
    a.ok = pooled_block(P, s, kPoolAppended, n_blk_iter, 0, a.j);
    a.t0 = max(0, a.j * P.g - P.pool_overlap);
    a.t1 = min(a.j * P.g + P.g, s.n_k);
    // every lane of the first 256 threads loads (tokens past the window re-read its last
    // one and are masked out when summed): no loaded register is merged with another
    // value, which would make the wavefront wait for the load here
    if (a.ok && act) {
#pragma unroll
        for (int u = 0; u < UN; u++) {
            const int t = a.t0 + u * TG + tg;
            const int tc = min(t, a.t1 - 1);
            const bool is_new = tc >= s.q0 && tc < s.q0 + s.n_q;
            const uint16_t *src = is_new ? k_new + ((s.q_off + (tc - s.q0)) * P.h_kv + c) * D
                                         : k + ((k_base + map.row(tc)) * P.h_kv + c) * D;
            a.raw[u] = reinterpret_cast<const uint4 *>(src)[chunk];
            a.valid |= t < a.t1 ? 1u << u : 0u;
        }
    }
    // the new token (one per sequence) is the block's own: its pieces go to the cache
    // (loaded once, outside the rounds, so no round's register waits for another's load)
    const int tn = s.q0;
    if (a.ok && act && s.n_q == 1 && tn >= a.j * P.g && tn < a.t1 && tg == (tn - a.t0) % TG) {
        const long long nrow = s.q_off * P.h_kv + c;
        knew = reinterpret_cast<const uint4 *>(k_new + nrow * D)[chunk];
        vnew = reinterpret_cast<const uint4 *>(v_new + nrow * D)[chunk];
        crow_new = (k_base + map.row(tn)) * P.h_kv + c;
    }
}

// sh: TG x D floats of LDS.  Every thread of the workgroup calls it.
template <int D, int UN, int POOL>
__device__ __forceinline__ void append_split_commit(const AppendSplit<D, UN> &a, const uint4 &knew,
                                                    const uint4 &vnew, long long crow_new, uint16_t *k, uint16_t *v,
                                                    float *sh)
{
    constexpr int L = D / 8, TG = 256 / L;
    const int tid = threadIdx.x, chunk = tid % L, tg = tid / L;
    if (!a.ok)
        return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < UN; u++) {
        const bool in = (a.valid >> u) & 1u;
        const uint32_t wv[4] = {in ? a.raw[u].x : 0u, in ? a.raw[u].y : 0u, in ? a.raw[u].z : 0u,
                                in ? a.raw[u].w : 0u};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            x[2 * i] = __uint_as_float(wv[i] << 16);
            x[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
        }
        float sc = 1.0f;
        if (POOL == 1) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++)
                ss += x[e] * x[e];
            ss = group_sum<L>(ss);
            sc = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            acc[e] += x[e] * sc;
    }
    if (tid < 256)
#pragma unroll
        for (int e = 0; e < 8; e++)
            sh[tg * D + chunk * 8 + e] = acc[e];
    if (crow_new >= 0) {
        reinterpret_cast<uint4 *>(k + crow_new * D)[chunk] = knew;
        reinterpret_cast<uint4 *>(v + crow_new * D)[chunk] = vnew;
    }
}

// After a barrier that follows append_split_commit.
template <int D, int UN, int POOL>
__device__ __forceinline__ void append_split_store(const KP &P, const AppendSplit<D, UN> &a, float *k_cmp, int b,
                                                   int c, const float *sh)
{
    constexpr int TG = 256 / (D / 8);
    const int tid = threadIdx.x;
    if (!a.ok || tid >= D)
        return;
    float sum = 0.f;
    for (int g2 = 0; g2 < TG; g2++)
        sum += sh[g2 * D + tid];
    if (POOL == 0)
        sum *= 1.0f / (float)(a.t1 - a.t0);
    k_cmp[(((long long)c * P.batch + b) * P.nb_max + a.j) * D + tid] = sum;
}

} // namespace sa
