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
#include "append_common.hpp"
#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

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

// The append's work items (append_common.hpp), one workgroup each.
template <typename T>
__global__ __launch_bounds__(256) void append_rows_kernel(KP P, const T *__restrict__ k_new,
                                                          const T *__restrict__ v_new, T *__restrict__ k,
                                                          T *__restrict__ v)
{
    append_rows_item<T>(P, k_new, v_new, k, v, blockIdx.x);
}

template <typename T, int D, int POOL>
__global__ __launch_bounds__(256) void append_pool_kernel(KP P, const T *__restrict__ k_new,
                                                          const T *__restrict__ v_new, T *__restrict__ k,
                                                          T *__restrict__ v, float *__restrict__ k_cmp, int n_blk_iter)
{
    append_pool_item<T, D, POOL>(P, k_new, v_new, k, v, k_cmp, n_blk_iter, blockIdx.x);
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
    const int n_blk = append_pool_blocks(P);
    const dim3 grid((unsigned)(P.batch * n_blk * P.h_kv));
    if (P.pool == 1)
        append_pool_kernel<T, D, 1><<<grid, dim3(256), 0, st>>>(P, (const T *)k_new, (const T *)v_new, (T *)k,
                                                                (T *)v, k_cmp, n_blk);
    else
        append_pool_kernel<T, D, 0><<<grid, dim3(256), 0, st>>>(P, (const T *)k_new, (const T *)v_new, (T *)k,
                                                                (T *)v, k_cmp, n_blk);
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
