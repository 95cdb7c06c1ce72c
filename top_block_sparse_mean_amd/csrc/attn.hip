// attn.hip -- attention restricted to the attended set, online softmax, fp32
// accumulation (PulseCol §3.1 Eq. (2): softmax of the logits with -inf outside
// the set; S3R review, sparse drafting formula: softmax and weighted sum over
// the retained keys only).
//
// The attended set of a query is walked in "position space": position pos of
// A(p) maps to a token through the selection row, which is read like a page
// table (init range, then the selected blocks clipped to the non-fixed region,
// then the window up to p).  Nothing is materialised.
//
// attn_valu: one workgroup per (query, KV head, chunk of <= HC query heads of
//   the group, split).  A key row is d/8 lanes x 16 B, so a wavefront reads
//   64/(d/8) rows per load; each lane group keeps its own running max / sum /
//   output for the tokens it saw; groups are merged through LDS at the end.
//   With more than one split, the partial (max, sum, unnormalised output) of
//   each split goes to the workspace and attn_combine merges them.
#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

template <typename T, int D, int HC>
__global__ __launch_bounds__(256) void attn_valu_kernel(KP P, const T *__restrict__ q, const T *__restrict__ k,
                                                        const T *__restrict__ v, const int32_t *__restrict__ idx,
                                                        const int32_t *__restrict__ n_idx, T *__restrict__ out,
                                                        float *__restrict__ lse, float *__restrict__ part,
                                                        int n_split, int n_hc)
{
    constexpr int L = D / 8;          // lanes per key row
    constexpr int TPI = 256 / L;      // key rows per workgroup iteration
    __shared__ float sh_m[TPI][HC], sh_l[TPI][HC];
    __shared__ float sh_o[TPI][HC][D];

    const long long unit = blockIdx.x;
    const int split = blockIdx.y;
    const int hc = (int)(unit % n_hc);
    const int c = (int)((unit / n_hc) % P.h_kv);
    const long long i = unit / ((long long)n_hc * P.h_kv);
    const int h0 = c * P.G + hc * HC;
    const int nh = min(HC, P.G - hc * HC);

    const int b = seq_of_query(P, i);
    const Seq s = seq_info(P, b);
    const int p = s.q0 + (int)(i - s.q_off);
    const long long row = P.shared ? b : i;
    const int p_sel = P.shared ? s.q0 - 1 : p;
    const int32_t *sel = idx + ((long long)c * P.rows + row) * P.topk;
    int nsel = n_idx[(long long)c * P.rows + row];
    nsel = clamp_nsel(P, nsel);
    const ASet a = aset_make(P, s.n_k, p, p_sel, sel, nsel);
    const long long k_base = kv_base(P, s);
    const KvMap kmap = kv_map(P, b);

    const int chunk = (a.total + n_split - 1) / n_split;
    const int s0 = split * chunk;
    const int s1 = min(a.total, s0 + chunk);

    const int tid = threadIdx.x, sub = tid % L, grp = tid / L;
    float qf[HC][8];
#pragma unroll
    for (int hh = 0; hh < HC; hh++) {
        if (hh < nh) {
            load8(q + (i * P.h_q + h0 + hh) * D + sub * 8, qf[hh]);
#pragma unroll
            for (int e = 0; e < 8; e++)
                qf[hh][e] *= P.scale_log2;
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                qf[hh][e] = 0.f;
        }
    }
    float m[HC], l[HC], o[HC][8];
#pragma unroll
    for (int hh = 0; hh < HC; hh++) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++)
            o[hh][e] = 0.f;
    }

    for (int base = s0; base < s1; base += 2 * TPI) {
        float kx[2][8], vx[2][8];
        bool ok[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            int pos = base + u * TPI + grp;
            ok[u] = pos < s1;
            if (ok[u]) {
                int t = aset_token(a, sel, pos);
                long long off = ((k_base + kmap.row(t)) * P.h_kv + c) * D + sub * 8;
                load8(k + off, kx[u]);
                load8(v + off, vx[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    kx[u][e] = vx[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
#pragma unroll
            for (int hh = 0; hh < HC; hh++) {
                float d0 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    d0 += qf[hh][e] * kx[u][e];
                float sc = group_sum<L>(d0);
                if (ok[u]) {
                    float mn = fmaxf(m[hh], sc);
                    float corr = exp2f(m[hh] - mn);
                    float pe = exp2f(sc - mn);
                    l[hh] = l[hh] * corr + pe;
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        o[hh][e] = o[hh][e] * corr + pe * vx[u][e];
                    m[hh] = mn;
                }
            }
        }
    }
    // merge the lane groups
#pragma unroll
    for (int hh = 0; hh < HC; hh++) {
        if (sub == 0) {
            sh_m[grp][hh] = m[hh];
            sh_l[grp][hh] = l[hh];
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            sh_o[grp][hh][sub * 8 + e] = o[hh][e];
    }
    __syncthreads();
    for (int it = tid; it < nh * D; it += 256) {
        int hh = it / D, e = it % D;
        float M = -INFINITY;
        for (int gq = 0; gq < TPI; gq++)
            M = fmaxf(M, sh_m[gq][hh]);
        float Ls = 0.f, O = 0.f;
        if (M > -INFINITY) {
            for (int gq = 0; gq < TPI; gq++) {
                float w = exp2f(sh_m[gq][hh] - M);
                Ls += sh_l[gq][hh] * w;
                O += sh_o[gq][hh][e] * w;
            }
        }
        const int h = h0 + hh;
        if (n_split == 1) {
            float val = O / Ls;
            if constexpr (sizeof(T) == 2)
                reinterpret_cast<uint16_t *>(out)[(i * P.h_q + h) * D + e] = f32_to_bf16(val);
            else
                out[(i * P.h_q + h) * D + e] = val;
            if (lse && e == 0)
                lse[(long long)h * P.total_q + i] = (M + log2f(Ls)) * 0.69314718055994531f;
        } else {
            float *dst = part + (((i * P.h_q + h) * n_split) + split) * (D + 2);
            dst[e] = O;
            if (e == 0) {
                dst[D] = M;
                dst[D + 1] = Ls;
            }
        }
    }
}

// Merge the splits of one (query, head): one wavefront each, 4 per workgroup.
// Lane s reads split s's (max, sum); the weights are broadcast from their lanes.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(KP P, const float *__restrict__ part, int n_split,
                                                           T *__restrict__ out, float *__restrict__ lse)
{
    const long long ih = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    if (ih >= P.total_q * P.h_q)
        return;
    const int lane = lane_id();
    const float *src = part + ih * n_split * (D + 2);
    float ms = lane < n_split ? src[lane * (D + 2) + D] : -INFINITY;
    float ls = lane < n_split ? src[lane * (D + 2) + D + 1] : 0.f;
    float M = ms;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        M = fmaxf(M, __shfl_xor(M, o, kWave));
    float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
    float Ls = ls * wgt;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        Ls += __shfl_xor(Ls, o, kWave);
    constexpr int EPL = D / kWave;
    float O[EPL];
#pragma unroll
    for (int x = 0; x < EPL; x++)
        O[x] = 0.f;
    for (int sp = 0; sp < n_split; sp++) {
        float f = __shfl(wgt, sp, kWave);
        const float *pp = src + sp * (D + 2);
#pragma unroll
        for (int x = 0; x < EPL; x++)
            O[x] += pp[lane + x * kWave] * f;
    }
    const long long i = ih / P.h_q;
    const int h = (int)(ih % P.h_q);
#pragma unroll
    for (int x = 0; x < EPL; x++) {
        float val = O[x] / Ls;
        long long o = ih * D + lane + x * kWave;
        if constexpr (sizeof(T) == 2)
            reinterpret_cast<uint16_t *>(out)[o] = f32_to_bf16(val);
        else
            out[o] = val;
    }
    if (lse && lane == 0)
        lse[(long long)h * P.total_q + i] = (M + log2f(Ls)) * 0.69314718055994531f;
}

static int head_chunk(const KP &P) { return P.G < 4 ? P.G : 4; }

int fwd_splits(const KP &P)
{
    if (wg_fwd_ok(P, P.dtype) || tile_fwd_ok(P, P.dtype))
        return 1;
    if (mfma_fwd_ok(P, P.dtype))
        return mfma_fwd_splits(P);
    long long a_max = (long long)P.n_init + (long long)P.topk * P.g + P.window + (P.shared ? P.max_q : 0);
    if (a_max > P.max_k)
        a_max = P.max_k;
    int hc = head_chunk(P);
    long long units = P.total_q * P.h_kv * ((P.G + hc - 1) / hc);
    long long by_len = (a_max + 255) / 256;
    long long by_fill = (4096 + units - 1) / units;
    long long sp = by_len < by_fill ? by_len : by_fill;
    if (sp > 32)
        sp = 32;
    return sp < 1 ? 1 : (int)sp;
}

template <typename T, int D>
static hipError_t launch_combine(const KP &P, const void *ws, int splits, void *out, float *lse, hipStream_t st)
{
    long long n = P.total_q * P.h_q;
    attn_combine_kernel<T, D><<<dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st>>>(P, (const float *)ws, splits,
                                                                                   (T *)out, lse);
    return hipGetLastError();
}

size_t fwd_workspace_bytes(const KP &P, int splits)
{
    if (splits <= 1)
        return 0;
    return (size_t)P.total_q * P.h_q * splits * (P.d + 2) * sizeof(float);
}

template <typename T, int D, int HC>
static hipError_t launch_fwd_t(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                               const int32_t *n_idx, void *out, float *lse, void *ws, int splits,
                               void *ev0, void *ev1, hipStream_t st)
{
    int n_hc = (P.G + HC - 1) / HC;
    long long units = P.total_q * P.h_kv * n_hc;
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    attn_valu_kernel<T, D, HC><<<dim3((unsigned)units, (unsigned)splits), dim3(256), 0, st>>>(
        P, (const T *)q, (const T *)k, (const T *)v, idx, n_idx, (T *)out, lse, (float *)ws, splits, n_hc);
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev1, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    return launch_combine<T, D>(P, ws, splits, out, lse, st);
}

template <typename T, int D>
static hipError_t launch_fwd_d(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                               const int32_t *n_idx, void *out, float *lse, void *ws, int splits, void *ev0,
                               void *ev1, hipStream_t st)
{
    switch (head_chunk(P)) {
    case 1: return launch_fwd_t<T, D, 1>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
    case 2: return launch_fwd_t<T, D, 2>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
    case 3: return launch_fwd_t<T, D, 3>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
    default: return launch_fwd_t<T, D, 4>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
    }
}

hipError_t launch_fwd(const KP &P, int dtype, const void *q, const void *k, const void *v, const int32_t *idx,
                      const int32_t *n_idx, void *out, float *lse, void *ws, int splits, void *ev0, void *ev1,
                      hipStream_t st)
{
    if (wg_fwd_ok(P, dtype))
        return launch_fwd_wg(P, q, k, v, idx, n_idx, out, lse, ev0, ev1, st);
    if (tile_fwd_ok(P, dtype))
        return launch_fwd_tile(P, q, k, v, idx, n_idx, out, lse, ev0, ev1, st);
    if (mfma_fwd_ok(P, dtype)) {
        hipError_t e = launch_fwd_mfma(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
        if (e != hipSuccess || splits == 1)
            return e;
        return P.d == 128 ? launch_combine<uint16_t, 128>(P, ws, splits, out, lse, st)
                          : launch_combine<uint16_t, 64>(P, ws, splits, out, lse, st);
    }
    if (dtype == 1)
        return P.d == 128 ? launch_fwd_d<uint16_t, 128>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st)
                          : launch_fwd_d<uint16_t, 64>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
    return P.d == 128 ? launch_fwd_d<float, 128>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st)
                      : launch_fwd_d<float, 64>(P, q, k, v, idx, n_idx, out, lse, ws, splits, ev0, ev1, st);
}

} // namespace sa
