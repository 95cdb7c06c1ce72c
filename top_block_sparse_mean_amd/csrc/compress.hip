// compress.hip -- pooled keys, one streaming pass over K.
//
// K~_j = mean of the keys of block j's pooling window (SparDA summary, Method:
// InfLLM-V2 pools keys by a parameter-free mean into overlapping compressed
// keys), or the sum of the L2-normalised keys (LSA deep-read, §2.2).  Block j
// is g consecutive tokens of one KV head, stride g; its window reaches
// pool_overlap tokens further back (clipped at token 0).
//
// Mapping: one thread owns 8 consecutive head-dim elements of one pooled
// vector.  Threads are numbered chunk-fastest, then KV head, then block, then
// sequence, so for a fixed token offset a wavefront reads d/8 x 16 B runs that
// are contiguous across KV heads (rows of K are [Hkv, d] contiguous): the
// pass is a coalesced stream of K and the kernel is HBM-bound.  L2SUM needs the
// norm of each key: its d/8 owners are adjacent lanes of one wavefront and sum
// their squares with xor shuffles; every lane runs the same g iterations so
// the shuffles stay converged.
#include "sa_common.hpp"
#include "sa_internal.hpp"

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

template <typename T, int D, int POOL>
__global__ __launch_bounds__(256) void compress_kernel(KP P, const T *__restrict__ k,
                                                       float *__restrict__ k_cmp, int n_blk_iter,
                                                       int mode)
{
    constexpr int L = D / 8;   // lanes per pooled vector
    long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    int chunk = (int)(tid % L);
    long long r = tid / L;
    int c = (int)(r % P.h_kv);
    r /= P.h_kv;
    int jj = (int)(r % n_blk_iter);
    int b = (int)(r / n_blk_iter);
    bool live = b < P.batch;
    int n_k = 0, j = 0;
    long long k_base = 0;
    KvMap map{nullptr, 0};
    if (live) {
        const Seq s = seq_info(P, b);
        n_k = s.n_k;
        k_base = kv_base(P, s);
        map = kv_map(P, b);
        live = pooled_block(P, s, mode, n_blk_iter, jj, j);
    }
    int t0 = max(0, j * P.g - P.pool_overlap);          // the block's pooling window [t0, t1)
    int t1 = min(j * P.g + P.g, n_k);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it = 0; it < P.g + P.pool_overlap; it++) {
        int t = t0 + it;
        bool ok = live && t < t1;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok)
            load8(k + ((k_base + map.row(t)) * P.h_kv + c) * D + chunk * 8, x);
        float s = 1.0f;
        if (POOL == 1) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++)
                ss += x[e] * x[e];
            ss = group_sum<L>(ss);
            s = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            acc[e] += x[e] * s;
    }
    if (!live)
        return;
    if (POOL == 0) {
        float inv = 1.0f / (float)(t1 - t0);
#pragma unroll
        for (int e = 0; e < 8; e++)
            acc[e] *= inv;
    }
    store8(k_cmp + (((long long)c * P.batch + b) * P.nb_max + j) * D + chunk * 8, acc);
}

// Few pooled vectors (a decode step re-pools the newest block of each
// sequence): one workgroup per (sequence, KV head, block); the block's tokens
// are spread over 256/(d/8) token groups and summed through LDS.
template <typename T, int D, int POOL>
__global__ __launch_bounds__(256) void compress_few_kernel(KP P, const T *__restrict__ k, float *__restrict__ k_cmp,
                                                           int n_blk_iter, int mode)
{
    constexpr int L = D / 8, TG = 256 / L;
    __shared__ float sh[TG][D];
    const int jj = blockIdx.x % n_blk_iter;
    const int c = (blockIdx.x / n_blk_iter) % P.h_kv;
    const int b = blockIdx.x / (n_blk_iter * P.h_kv);
    const int tid = threadIdx.x, chunk = tid % L, tg = tid / L;
    const Seq s = seq_info(P, b);
    const long long k_base = kv_base(P, s);
    const KvMap map = kv_map(P, b);
    const int n_k = s.n_k;
    int j;
    if (!pooled_block(P, s, mode, n_blk_iter, jj, j))
        return;
    const int t0 = max(0, j * P.g - P.pool_overlap), t1 = min(j * P.g + P.g, n_k);   // pooling window
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it = 0; it < P.g + P.pool_overlap; it += TG) {
        int t = t0 + it + tg;
        bool ok = t < t1;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok)
            load8(k + ((k_base + map.row(t)) * P.h_kv + c) * D + chunk * 8, x);
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
}

template <typename T, int D>
static hipError_t launch_compress_t(const KP &P, const void *k, float *k_cmp, int n_blk_iter, int mode,
                                    hipStream_t st)
{
    long long vectors = (long long)P.batch * n_blk_iter * P.h_kv;
    if (vectors <= 4096 && P.g >= 16) {          // too few vectors to fill the chip one thread-slice each
        dim3 grid((unsigned)vectors);
        if (P.pool == 1)
            compress_few_kernel<T, D, 1><<<grid, dim3(256), 0, st>>>(P, (const T *)k, k_cmp, n_blk_iter, mode);
        else
            compress_few_kernel<T, D, 0><<<grid, dim3(256), 0, st>>>(P, (const T *)k, k_cmp, n_blk_iter, mode);
        return hipGetLastError();
    }
    long long threads = vectors * (D / 8);
    long long blocks = (threads + 255) / 256;
    if (P.pool == 1)
        compress_kernel<T, D, 1><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
            P, (const T *)k, k_cmp, n_blk_iter, mode);
    else
        compress_kernel<T, D, 0><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
            P, (const T *)k, k_cmp, n_blk_iter, mode);
    return hipGetLastError();
}

static hipError_t launch_pool(const KP &P, int dtype, const void *k, float *k_cmp, int n_blk_iter, int mode,
                              hipStream_t st)
{
    if (dtype == 1)
        return P.d == 128 ? launch_compress_t<uint16_t, 128>(P, k, k_cmp, n_blk_iter, mode, st)
                          : launch_compress_t<uint16_t, 64>(P, k, k_cmp, n_blk_iter, mode, st);
    return P.d == 128 ? launch_compress_t<float, 128>(P, k, k_cmp, n_blk_iter, mode, st)
                      : launch_compress_t<float, 64>(P, k, k_cmp, n_blk_iter, mode, st);
}

hipError_t launch_compress(const KP &P, int dtype, const void *k, float *k_cmp, int n_tail, hipStream_t st)
{
    int n_blk_iter = n_tail > 0 ? (n_tail < P.nb_max ? n_tail : P.nb_max) : P.nb_max;
    return launch_pool(P, dtype, k, k_cmp, n_blk_iter, n_tail > 0 ? kPoolTail : kPoolAll, st);
}

// ---------------------------------------------------------------- append

// Copy of one token's 16-byte piece: k_new / v_new row i -> cache row `row`.
template <typename T>
__device__ __forceinline__ void copy_piece(const T *src, T *dst, long long src_row, long long dst_row, int width,
                                           int x)
{
    reinterpret_cast<uint4 *>(dst + dst_row * width)[x] = reinterpret_cast<const uint4 *>(src + src_row * width)[x];
}

// No pooling (g = 1 or no pooled keys): one workgroup per new token row i copies
// its h_kv x d keys and values to the cache row of position q0_b + (i - q_off).
template <typename T>
__global__ __launch_bounds__(256) void append_rows_kernel(KP P, const T *__restrict__ k_new,
                                                          const T *__restrict__ v_new, T *__restrict__ k,
                                                          T *__restrict__ v)
{
    const long long i = blockIdx.x;
    const int b = seq_of_query(P, i);
    const Seq s = seq_info(P, b);
    const long long row = kv_base(P, s) + kv_map(P, b).row(s.q0 + (int)(i - s.q_off));
    const int width = P.h_kv * P.d, pieces = width * (int)sizeof(T) / 16;
    for (int x = threadIdx.x; x < pieces; x += blockDim.x) {
        copy_piece(k_new, k, i, row, width, x);
        copy_piece(v_new, v, i, row, width, x);
    }
}

// With pooling: one workgroup per (sequence, KV head, block whose pooling window
// holds a new token).  New tokens in the window are taken from k_new / v_new
// (and written to the cache when they belong to the block itself); its other
// tokens are read from the cache; the window is pooled exactly as
// compress_few_kernel pools it.  Each new (token, head) belongs to one block, so
// every cache row is written by one workgroup, and no workgroup reads a row
// another writes.
template <typename T, int D, int POOL>
__global__ __launch_bounds__(256) void append_pool_kernel(KP P, const T *__restrict__ k_new,
                                                          const T *__restrict__ v_new, T *__restrict__ k,
                                                          T *__restrict__ v, float *__restrict__ k_cmp, int n_blk_iter)
{
    constexpr int L = D / 8, TG = 256 / L;
    __shared__ float sh[TG][D];
    const int jj = blockIdx.x % n_blk_iter;
    const int c = (blockIdx.x / n_blk_iter) % P.h_kv;
    const int b = blockIdx.x / (n_blk_iter * P.h_kv);
    const int tid = threadIdx.x, chunk = tid % L, tg = tid / L;
    const Seq s = seq_info(P, b);
    const long long k_base = kv_base(P, s);
    const KvMap map = kv_map(P, b);
    int j;
    if (!pooled_block(P, s, kPoolAppended, n_blk_iter, jj, j))
        return;
    const int t0 = max(0, j * P.g - P.pool_overlap), t1 = min(j * P.g + P.g, s.n_k);   // pooling window
    // UN token rounds of the window are loaded before any is summed (the window of a
    // 64-token block is 4 rounds: one memory latency instead of four); the sums run
    // in token-round order as without the batching.
    constexpr int UN = 4;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int it0 = 0; it0 < P.g + P.pool_overlap; it0 += UN * TG) {
        float x[UN][8];
#pragma unroll
        for (int u = 0; u < UN; u++) {
            const int t = t0 + it0 + u * TG + tg;
#pragma unroll
            for (int e = 0; e < 8; e++)
                x[u][e] = 0.f;
            if (t < t1) {
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
}

template <typename T, int D>
static hipError_t launch_append_t(const KP &P, const void *k_new, const void *v_new, void *k, void *v,
                                  float *k_cmp, hipStream_t st)
{
    if (!k_cmp || P.g == 1) {
        append_rows_kernel<T><<<dim3((unsigned)P.total_q), dim3(256), 0, st>>>(P, (const T *)k_new,
                                                                             (const T *)v_new, (T *)k, (T *)v);
        return hipGetLastError();
    }
    // M consecutive tokens lie in the windows of at most ceil((M + o) / g) + 1 blocks
    long long n_blk = ((long long)P.max_q + P.pool_overlap + P.g - 1) / P.g + 1;
    if (n_blk > P.nb_max)
        n_blk = P.nb_max;
    const dim3 grid((unsigned)(P.batch * n_blk * P.h_kv));
    if (P.pool == 1)
        append_pool_kernel<T, D, 1><<<grid, dim3(256), 0, st>>>(P, (const T *)k_new, (const T *)v_new, (T *)k,
                                                                (T *)v, k_cmp, (int)n_blk);
    else
        append_pool_kernel<T, D, 0><<<grid, dim3(256), 0, st>>>(P, (const T *)k_new, (const T *)v_new, (T *)k,
                                                                (T *)v, k_cmp, (int)n_blk);
    return hipGetLastError();
}

hipError_t launch_append(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                         float *k_cmp, hipStream_t st)
{
    if (dtype == 1)
        return P.d == 128 ? launch_append_t<uint16_t, 128>(P, k_new, v_new, k, v, k_cmp, st)
                          : launch_append_t<uint16_t, 64>(P, k_new, v_new, k, v, k_cmp, st);
    return P.d == 128 ? launch_append_t<float, 128>(P, k_new, v_new, k, v, k_cmp, st)
                      : launch_append_t<float, 64>(P, k_new, v_new, k, v, k_cmp, st);
}

} // namespace sa
