// attn_decode.hip -- bf16 sparse attention on gfx950 matrix cores for units of
// up to 16 query rows that share one attended set: the GQA heads of one query
// (per-query selection), or every head of every draft of a sequence (shared
// selection; drafts differ only by their causal limit).  The next chunk's K/V
// loads are issued before the current chunk is computed.  The attended
// positions of the workgroup's split are first mapped to K/V rows into LDS (the
// selection row, and for a paged cache the block table, read like page tables).
// Splits write (max, sum, unnormalised output) partials that attn_combine merges.
#include "mfma_common.hpp"

namespace sa {

// grid: (units * h_kv, splits); 256 threads.  unit = query (per-query selection) or sequence (shared).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(KP P, const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v,
                                                           const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ n_idx,
                                                           uint16_t *__restrict__ out, float *__restrict__ lse,
                                                           float *__restrict__ part, int n_split)
{
    constexpr int KS = D / 32;
    __shared__ int sh_tok[kTokCap];            // token list; reused for the wave merge
    __shared__ int sh_sel[kSelCap];            // the unit's selection row
    __shared__ float sh_m[4][16], sh_l[4][16];
    const int c = blockIdx.x % P.h_kv;
    const long long u = blockIdx.x / P.h_kv;
    const int split = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rr = lane & 15, g4 = lane >> 4;
    // the selection row is known from the unit alone: start its loads first
    const long long row0 = u;                 // query (per-query selection) or sequence (shared)
    const int32_t *sel_g = idx + ((long long)c * P.rows + row0) * P.topk;
    const bool sel_in_lds = P.topk <= kSelCap;
    if (sel_in_lds)
        for (int x = tid; x < P.topk; x += 256)
            sh_sel[x] = sel_g[x];
    int nsel = n_idx[(long long)c * P.rows + row0];

    int b, p_sel, p_max;
    long long q_first, row;
    int nq_u;
    if (P.shared) {
        b = (int)u;
        row = b;
    } else {
        b = seq_of_query(P, u);
        row = u;
    }
    const Seq s = seq_info(P, b);
    if (P.shared) {
        q_first = s.q_off;
        nq_u = s.n_q;
        p_sel = s.q0 - 1;
        p_max = s.q0 + s.n_q - 1;
    } else {
        q_first = u;
        nq_u = 1;
        p_max = s.q0 + (int)(u - s.q_off);
        p_sel = p_max;
    }
    const int R = nq_u * P.G;                 // <= 16 (checked by the host)
    (void)row;
    nsel = clamp_nsel(P, nsel);
    __syncthreads();                          // sh_sel complete
    const int32_t *sel = sel_in_lds ? sh_sel : sel_g;
    const ASet a = aset_make(P, s.n_k, p_max, p_sel, sel, nsel);
    const int chunk = (a.total + n_split - 1) / n_split;
    const int s0 = split * chunk;
    const int n = max(0, min(a.total, s0 + chunk) - s0);
    const KvMap kmap = kv_map(P, b);
    for (int x = tid; x < n; x += 256)
        sh_tok[x] = kmap.row(aset_token(a, sel, s0 + x));

    // B operand of S^T = K Q^T: lane l holds Q[row l%16][32 ks + 8 (l/16) .. +8]
    bf16x8 qop[KS];
    int lim = 0;                              // live list entries of this lane's row (split-local)
    if (rr < R) {
        const long long qi = q_first + rr / P.G;
        const int h = c * P.G + rr % P.G;
        const uint16_t *qp = q + (qi * P.h_q + h) * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
        const int p_row = s.q0 + (int)(q_first - s.q_off) + rr / P.G;
        lim = a.total - s0 - (p_max - p_row);
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();

    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (kv_base(P, s) * P.h_kv + c) * D;
    const uint16_t *vb = v + (kv_base(P, s) * P.h_kv + c) * D;
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int p = 0; p < 8; p++)
        acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

    ChunkRegs<D> ra, rb;
    if (32 * w < n)
        load_chunk<D>(ra, sh_tok, 32 * w, n, kb, vb, tstride, rr, g4, lim);
    for (int ch = w; 32 * ch < n; ch += 8) {
        const int c1 = ch + 4;
        if (32 * c1 < n)
            load_chunk<D>(rb, sh_tok, 32 * c1, n, kb, vb, tstride, rr, g4, lim);
        compute_chunk<D>(ra, ra.live, qop, P.scale_log2, g4, m_run, l_part, acc);
        if (32 * c1 >= n)
            break;
        const int c2 = c1 + 4;
        if (32 * c2 < n)
            load_chunk<D>(ra, sh_tok, 32 * c2, n, kb, vb, tstride, rr, g4, lim);
        compute_chunk<D>(rb, rb.live, qop, P.scale_log2, g4, m_run, l_part, acc);
    }
    float l_row = l_part + __shfl_xor(l_part, 16, kWave);
    l_row += __shfl_xor(l_row, 32, kWave);
    __syncthreads();                           // every wave is done with the token list
    float *sh_o = reinterpret_cast<float *>(sh_tok);    // [4 waves][16 rows][D]
    if (g4 == 0) {
        sh_m[w][rr] = m_run;
        sh_l[w][rr] = l_row;
    }
    if (D == 128 || rr < D / 8) {
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
            float *dst = sh_o + (w * 16 + 4 * g4 + qq) * D + 8 * rr;
#pragma unroll
            for (int p = 0; p < 8; p++)
                dst[p] = acc[p][qq];
        }
    }
    __syncthreads();
    for (int it = tid; it < R * D; it += 256) {
        const int r = it / D, e = it % D;
        float M = fmaxf(fmaxf(sh_m[0][r], sh_m[1][r]), fmaxf(sh_m[2][r], sh_m[3][r]));
        float Ls = 0.f, O = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < 4; ww++) {
                float f = exp2f(sh_m[ww][r] - M);
                Ls += sh_l[ww][r] * f;
                O += sh_o[(ww * 16 + r) * D + e] * f;
            }
        }
        const long long qi = q_first + r / P.G;
        const int h = c * P.G + r % P.G;
        if (n_split == 1) {
            out[(qi * P.h_q + h) * D + e] = f32_to_bf16(O / Ls);
            if (lse && e == 0)
                lse[(long long)h * P.total_q + qi] = (M + log2f(Ls)) * 0.69314718055994531f;
        } else {
            float *dst = part + ((qi * P.h_q + h) * n_split + split) * (D + 2);
            dst[e] = O;
            if (e == 0) {
                dst[D] = M;
                dst[D + 1] = Ls;
            }
        }
    }
}

// Largest attended set of any unit (init + selected blocks + window, plus the
// drafts of a shared selection), bounded by the longest cache.
static long long mfma_set_max(const KP &P)
{
    long long a_max = (long long)P.n_init + (long long)P.topk * P.g + P.window + (P.shared ? P.max_q : 0);
    return a_max > P.max_k ? P.max_k : a_max;
}

// The gather kernel keeps each split's token list in LDS (kTokCap entries) and
// the combine merges at most kMaxSplits splits, so it serves sets of at most
// kMaxSplits * kTokCap tokens; longer sets take the VALU kernel, which walks
// the set's positions with no list.
bool mfma_fwd_ok(const KP &P, int dtype)
{
    if (dtype != 1)
        return false;
    long long rows = P.shared ? (long long)P.max_q * P.G : P.G;
    return rows <= 16 && mfma_set_max(P) <= (long long)kMaxSplits * kTokCap;
}

int mfma_fwd_splits(const KP &P)
{
    const long long a_max = mfma_set_max(P);
    long long units = (P.shared ? P.batch : P.total_q) * P.h_kv;
    long long need = (a_max + kTokCap - 1) / kTokCap;          // the token list must fit in LDS
    long long fill = (256 + units - 1) / units;                // at least one workgroup per CU
    long long by_len = (a_max + 255) / 256;                    // >= 2 chunks per wavefront
    long long sp = fill < by_len ? fill : by_len;
    if (sp < need)
        sp = need;
    if (const char *e = getenv("SPARSE_ATTN_FWD_SPLITS")) {     // tuning override
        int v = atoi(e);
        if (v > 0)
            sp = v > need ? v : need;
    }
    if (sp > kMaxSplits)                                       // need <= kMaxSplits (mfma_fwd_ok)
        sp = kMaxSplits;
    return sp < 1 ? 1 : (int)sp;
}

hipError_t launch_fwd_mfma(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                           const int32_t *n_idx, void *out, float *lse, void *ws, int splits, void *ev0, void *ev1,
                           hipStream_t st)
{
    long long units = (P.shared ? P.batch : P.total_q) * P.h_kv;
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    if (P.d == 128)
        attn_mfma_kernel<128><<<dim3((unsigned)units, (unsigned)splits), dim3(256), 0, st>>>(
            P, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
            (float *)ws, splits);
    else
        attn_mfma_kernel<64><<<dim3((unsigned)units, (unsigned)splits), dim3(256), 0, st>>>(
            P, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
            (float *)ws, splits);
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev1, st);
    return hipGetLastError();
}

} // namespace sa
