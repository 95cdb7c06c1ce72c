// attn_mfma.hip -- bf16 sparse attention on gfx950 matrix cores for units of
// up to 16 query rows that share one attended set: the GQA heads of one query
// (per-query selection), or every head of every draft of a sequence (shared
// selection; drafts differ only by their causal limit).  Online softmax with
// fp32 running max / sum / output (PulseCol §3.1 Eq. (2); S3R review, sparse
// drafting formula).
//
// Per wavefront, 32 attended positions at a time:
//   S^T = K Q^T   two 16x16x32 bf16 MFMA tiles per k-step (16 tokens x 16 rows);
//                 A = K rows loaded straight from HBM (lane l: token l%16, 16 B
//                 of the head dimension), B = Q^T kept in registers.
//   P   = softmax numerators, fp32 -> bf16 in the layout the next MFMA reads as
//         its A operand (the 8 logits a lane holds are the 8 tokens its A row needs).
//   O   += P V    eight 16x16x32 tiles; B = V loaded straight from HBM as one
//                 256 B row per 16 lanes, transposed 8x8 in registers with
//                 v_perm, output column n of tile p is head-dim index 8n + p.
// The next chunk's K/V loads are issued before the current chunk is computed.
// The attended positions of the workgroup's split are first mapped to tokens
// into LDS (the selection row is read like a page table).  Splits write
// (max, sum, unnormalised output) partials that attn_combine merges.
#include <stdlib.h>

#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D>
struct ChunkRegs {
    u32x4 k[2][D / 32];   // K rows of the two 16-token subtiles, A-operand layout
    u32x4 v[8];           // V rows of the lane's 8 tokens, head-dim slice 8*(l%16) .. +8
    uint32_t live;        // bit i: logit i of this lane is inside the split and causal for its row
};

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

template <int D>
__device__ __forceinline__ void load_chunk(ChunkRegs<D> &r, const int *tok, int base, int n, const uint16_t *kb,
                                           const uint16_t *vb, long long tstride, int rr, int g4, int p_row)
{
    constexpr int KS = D / 32;
#pragma unroll
    for (int s = 0; s < 2; s++) {
        int pos = min(base + 16 * s + rr, n - 1);
        long long off = (long long)tok[pos] * tstride + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            r.k[s][ks] = ld16(kb + off + 32 * ks);
    }
    r.live = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int pos = base + (i < 4 ? 4 * g4 + i : 16 + 4 * g4 + (i - 4));
        int t = tok[min(pos, n - 1)];
        r.live |= (pos < n && t <= p_row) ? (1u << i) : 0u;
        if (D == 128 || rr < D / 8)
            r.v[i] = ld16(vb + (long long)t * tstride + 8 * rr);
        else
            r.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int D>
__device__ __forceinline__ void compute_chunk(const ChunkRegs<D> &r, uint32_t live, const bf16x8 (&qop)[D / 32],
                                              float scale_log2, int g4, float &m_run, float &l_part, f32x4 (&acc)[8])
{
    constexpr int KS = D / 32;
    f32x4 st[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
        st[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            st[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[s][ks]), qop[ks],
                                                            st[s], 0, 0, 0);
    }
    float sv[8];
    float mc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float x = st[i >> 2][i & 3] * scale_log2;
        sv[i] = (live >> i) & 1u ? x : -INFINITY;
        mc = fmaxf(mc, sv[i]);
    }
    mc = fmaxf(mc, __shfl_xor(mc, 16, kWave));
    mc = fmaxf(mc, __shfl_xor(mc, 32, kWave));
    const float m_new = fmaxf(m_run, mc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float sum = 0.f;
    bf16x8 aop;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float pe = exp2f(sv[i] - m_use);
        sum += pe;
        aop[i] = (__bf16)pe;
    }
    l_part = l_part * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        float a = __shfl(alpha, 4 * g4 + q, kWave);
#pragma unroll
        for (int p = 0; p < 8; p++)
            acc[p][q] *= a;
    }
#pragma unroll
    for (int p = 0; p < 8; p++) {
        const uint32_t sel = (p & 1) ? 0x07060302u : 0x05040100u;
        u32x4 b;
#pragma unroll
        for (int w = 0; w < 4; w++)
            b[w] = __builtin_amdgcn_perm(r.v[2 * w + 1][p >> 1], r.v[2 * w][p >> 1], sel);
        acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, __builtin_bit_cast(bf16x8, b), acc[p], 0, 0, 0);
    }
}

constexpr int kTokCap = 8192;

// Exclusive scan of one int per thread over a 512-thread workgroup; (exclusive, total).
__device__ __forceinline__ int2 block_scan_int_512(int v, int *sh)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(incl, o, kWave);
        if (lane >= o)
            incl += t;
    }
    if (lane == kWave - 1)
        sh[w] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int c = sh[i];
        off += i < w ? c : 0;
        tot += c;
    }
    __syncthreads();
    return make_int2(off + incl - v, tot);
}
constexpr int kSelCap = 4096;

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
    nsel = nsel < 0 ? 0 : (nsel > P.topk ? P.topk : nsel);
    __syncthreads();                          // sh_sel complete
    const int32_t *sel = sel_in_lds ? sh_sel : sel_g;
    const ASet a = aset_make(P, s.n_k, p_max, p_sel, sel, nsel);
    const int chunk = (a.total + n_split - 1) / n_split;
    const int s0 = split * chunk;
    const int n = max(0, min(a.total, s0 + chunk) - s0);
    for (int x = tid; x < n; x += 256)
        sh_tok[x] = aset_token(a, sel, s0 + x);

    // B operand of S^T = K Q^T: lane l holds Q[row l%16][32 ks + 8 (l/16) .. +8]
    bf16x8 qop[KS];
    int p_row = -1;
    if (rr < R) {
        const long long qi = q_first + rr / P.G;
        const int h = c * P.G + rr % P.G;
        const uint16_t *qp = q + (qi * P.h_q + h) * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
        p_row = s.q0 + (int)(q_first - s.q_off) + rr / P.G;
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();

    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (s.k_off * P.h_kv + c) * D;
    const uint16_t *vb = v + (s.k_off * P.h_kv + c) * D;
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int p = 0; p < 8; p++)
        acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

    ChunkRegs<D> ra, rb;
    if (32 * w < n)
        load_chunk<D>(ra, sh_tok, 32 * w, n, kb, vb, tstride, rr, g4, p_row);
    for (int ch = w; 32 * ch < n; ch += 8) {
        const int c1 = ch + 4;
        if (32 * c1 < n)
            load_chunk<D>(rb, sh_tok, 32 * c1, n, kb, vb, tstride, rr, g4, p_row);
        compute_chunk<D>(ra, ra.live, qop, P.scale_log2, g4, m_run, l_part, acc);
        if (32 * c1 >= n)
            break;
        const int c2 = c1 + 4;
        if (32 * c2 < n)
            load_chunk<D>(ra, sh_tok, 32 * c2, n, kb, vb, tstride, rr, g4, p_row);
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

// ---------------------------------------------------------------- union tiles (prefill)

// Load one 32-token key tile starting at token t0 (contiguous), with the lane's
// 8-bit live mask taken from the 32-bit token mask of its row.
template <int D>
__device__ __forceinline__ void load_tile(ChunkRegs<D> &r, int t0, int n_k, uint32_t m32, const uint16_t *kb,
                                          const uint16_t *vb, long long tstride, int rr, int g4)
{
    constexpr int KS = D / 32;
#pragma unroll
    for (int s = 0; s < 2; s++) {
        int t = min(t0 + 16 * s + rr, n_k - 1);
        long long off = (long long)t * tstride + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            r.k[s][ks] = ld16(kb + off + 32 * ks);
    }
    r.live = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int off = i < 4 ? 4 * g4 + i : 16 + 4 * g4 + (i - 4);
        int t = min(t0 + off, n_k - 1);
        r.live |= ((m32 >> off) & 1u) << i;
        if (D == 128 || rr < D / 8)
            r.v[i] = ld16(vb + (long long)t * tstride + 8 * rr);
        else
            r.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Tokens [t0, t0+32) of a query at p with window start lo_w and the tile's
// selected bit: causal & (init | window | selected block).
__device__ __forceinline__ uint32_t tile_mask(int t0, int p, int n_init, int lo_w, bool sel)
{
    auto below = [](int n) -> uint32_t {      // bits [0, n) for n clamped to [0, 32]
        return n <= 0 ? 0u : (n >= 32 ? 0xffffffffu : ((1u << n) - 1u));
    };
    uint32_t causal = below(p - t0 + 1);
    uint32_t init = below(n_init - t0);
    uint32_t win = ~below(lo_w - t0);
    return causal & (init | win | (sel ? 0xffffffffu : 0u));
}

constexpr int kTileWaves = 4;
constexpr int kTileMax = 4096;             // 32-token tiles per sequence (max_k <= 131072)
constexpr int kTileWords = kTileMax / 32;

// grid: 1-D, n_qtile * batch * h_kv workgroups, remapped so that each XCD
// (blockIdx % 8) works through a contiguous range of (sequence, KV head, query
// tile) items.  Wavefront w owns 16/G consecutive queries = 16 rows.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_tile_kernel(KP P, const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v,
                                                           const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ n_idx,
                                                           uint16_t *__restrict__ out, float *__restrict__ lse,
                                                           int n_qtile)
{
    constexpr int KS = D / 32;
    __shared__ uint32_t sh_sel[kTileWaves][4][kTileWords];   // per-query selected-tile bits (G >= 4)
    __shared__ uint32_t sh_uni[kTileWaves][kTileWords];
    __shared__ int sh_list[kTileWaves][kTileMax];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rr = lane & 15, g4 = lane >> 4;
    // XCD-contiguous work mapping
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    const long long per_xcd = (n_items + 7) / 8;
    const long long item = (long long)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= n_items)
        return;
    const int qt = (int)(item % n_qtile);
    const int c = (int)((item / n_qtile) % P.h_kv);
    const int b = (int)(item / ((long long)n_qtile * P.h_kv));
    const Seq s = seq_info(P, b);
    const int QPW = 16 / P.G;                       // queries per wavefront (<= 4)
    const int qw0 = qt * kTileWaves * QPW + w * QPW;    // first local query of this wave
    const int nqw = max(0, min(QPW, s.n_q - qw0));
    const int ntile = (s.n_k + 31) / 32;
    const int nword = (ntile + 31) / 32;
    for (int x = lane; x < 4 * kTileWords; x += kWave)
        (&sh_sel[w][0][0])[x] = 0u;
    for (int x = lane; x < kTileWords; x += kWave)
        sh_uni[w][x] = 0u;
    __syncthreads();
    // selected tiles of each query of the wave
    const int tpb = P.g / 32;                       // tiles per pooled block
    for (int qq = 0; qq < nqw; qq++) {
        const long long qi = s.q_off + qw0 + qq;
        const int32_t *sel = idx + ((long long)c * P.rows + qi) * P.topk;
        int ns = n_idx[(long long)c * P.rows + qi];
        ns = ns < 0 ? 0 : (ns > P.topk ? P.topk : ns);
        for (int e = lane; e < ns * tpb; e += kWave) {
            int tile = sel[e / tpb] * tpb + e % tpb;
            if (tile >= 0 && tile < ntile) {
                atomicOr(&sh_sel[w][qq][tile >> 5], 1u << (tile & 31));
                atomicOr(&sh_uni[w][tile >> 5], 1u << (tile & 31));
            }
        }
    }
    // init and window tiles of the wave's queries
    int p_first = s.q0 + qw0, p_last = s.q0 + qw0 + nqw - 1;
    if (nqw > 0) {
        int lo_first = max(P.n_init, p_first - P.window + 1);
        int i_hi = (min(P.n_init, p_last + 1) + 31) / 32;          // init tiles [0, i_hi)
        for (int tile = lane; tile < i_hi; tile += kWave)
            atomicOr(&sh_uni[w][tile >> 5], 1u << (tile & 31));
        for (int tile = lo_first / 32 + lane; tile <= p_last / 32; tile += kWave)
            atomicOr(&sh_uni[w][tile >> 5], 1u << (tile & 31));
    }
    __syncthreads();
    // compact the union into an ascending tile list
    int n_list = 0;
    for (int base = 0; base < nword; base += kWave) {
        int wd = base + lane;
        uint32_t bits = wd < nword ? sh_uni[w][wd] : 0u;
        int cnt = __popc(bits);
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            int t = __shfl_up(incl, o, kWave);
            if (lane >= o)
                incl += t;
        }
        int pos = n_list + incl - cnt;
        while (bits) {
            int bit = __ffs(bits) - 1;
            bits &= bits - 1;
            sh_list[w][pos++] = wd * 32 + bit;
        }
        n_list += __shfl(incl, kWave - 1, kWave);
    }
    __syncthreads();

    // this lane's row: query qq = rr / G, head c*G + rr % G
    const int qq = rr / P.G;
    const bool row_ok = qq < nqw;
    const long long qi = s.q_off + qw0 + (row_ok ? qq : 0);
    const int p_row = row_ok ? s.q0 + qw0 + qq : -1;
    const int lo_w = max(P.n_init, p_row - P.window + 1);
    bf16x8 qop[KS];
    if (row_ok) {
        const uint16_t *qp = q + (qi * P.h_q + c * P.G + rr % P.G) * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const uint32_t *selw = sh_sel[w][row_ok ? qq : 0];
    auto row_mask = [&](int tile) -> uint32_t {
        if (!row_ok)
            return 0u;
        bool sb = (selw[tile >> 5] >> (tile & 31)) & 1u;
        return tile_mask(tile * 32, p_row, P.n_init, lo_w, sb);
    };
    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (s.k_off * P.h_kv + c) * D;
    const uint16_t *vb = v + (s.k_off * P.h_kv + c) * D;
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int p = 0; p < 8; p++)
        acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    ChunkRegs<D> ra, rb;
    if (n_list > 0) {
        int t = sh_list[w][0];
        load_tile<D>(ra, t * 32, s.n_k, row_mask(t), kb, vb, tstride, rr, g4);
    }
    for (int it = 0; it < n_list; it += 2) {
        if (it + 1 < n_list) {
            int t = sh_list[w][it + 1];
            load_tile<D>(rb, t * 32, s.n_k, row_mask(t), kb, vb, tstride, rr, g4);
        }
        compute_chunk<D>(ra, ra.live, qop, P.scale_log2, g4, m_run, l_part, acc);
        if (it + 1 >= n_list)
            break;
        if (it + 2 < n_list) {
            int t = sh_list[w][it + 2];
            load_tile<D>(ra, t * 32, s.n_k, row_mask(t), kb, vb, tstride, rr, g4);
        }
        compute_chunk<D>(rb, rb.live, qop, P.scale_log2, g4, m_run, l_part, acc);
    }
    float l_row = l_part + __shfl_xor(l_part, 16, kWave);
    l_row += __shfl_xor(l_row, 32, kWave);
    // output: lane (g4 group) holds rows 4*g4 + r4, head-dim 8*rr + p; the row's
    // (max, sum) live in lanes with lane%16 == row
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
        const int row = 4 * g4 + r4;
        const float lrow = __shfl(l_row, row, kWave);
        const float mrow = __shfl(m_run, row, kWave);
        const int rq = row / P.G;
        if (rq < nqw && (D == 128 || rr < D / 8)) {
            const long long oq = s.q_off + qw0 + rq;
            const int h = c * P.G + row % P.G;
            const float inv = 1.0f / lrow;
            float o8[8];
#pragma unroll
            for (int p = 0; p < 8; p++)
                o8[p] = acc[p][r4] * inv;
            store8(out + (oq * P.h_q + h) * D + 8 * rr, o8);
            if (lse && rr == 0)
                lse[(long long)h * P.total_q + oq] = (mrow + log2f(lrow)) * 0.69314718055994531f;
        }
    }
}

// ---------------------------------------------------------------- shared union tiles (prefill)

// 8 wavefronts share each 64-token K/V tile through LDS.  A workgroup owns 8 x
// 32/G consecutive queries (64 for G = 4); wavefront w owns 32 rows (two 16-row
// MFMA tiles) = 32/G queries x G heads.  The workgroup's tile list is the union
// of its queries' init tiles, windows and selected blocks (block = tile, g = 64);
// for each listed tile a 64-bit mask says which of its queries selected it.  The
// list is walked in lockstep: while tile e is computed from LDS, the loads of
// tile e + kWgStage are in flight in registers and tile e + 1 is written to the
// other LDS buffer at the end of the iteration (one barrier per tile).  A
// wavefront skips the MFMA work of tiles none of its rows attends.
constexpr int kWgWaves = 8;
constexpr int kWgQueries = 64;                 // 8 waves x 8 queries (G = 4)
constexpr int kWgMaxTiles = 2048;              // 64-token tiles per sequence (max_k <= 131072)
constexpr int kWgStage = 2;                    // tiles in flight in registers
constexpr int kWgPitch = 272;                  // LDS bytes per staged 256-byte row (bank spread)

struct WgStage {
    u32x4 c[4];                                // this thread's 4 x 16 B of a 32 KB K/V tile
};

__device__ __forceinline__ void wg_issue(WgStage &st, const uint16_t *kb, const uint16_t *vb, long long tstride,
                                         int t0, int n_k, int tid)
{
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int chunk = tid + 512 * u;       // 2048 chunks: 128 rows (64 K, 64 V) x 16
        const int row = chunk >> 4, col = chunk & 15;
        const int t = min(max(t0 + (row & 63), 0), n_k - 1);
        const uint16_t *base = row < 64 ? kb : vb;
        st.c[u] = ld16(base + (long long)t * tstride + 8 * col);
    }
}

__device__ __forceinline__ void wg_write(const WgStage &st, unsigned char *buf, int tid)
{
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int chunk = tid + 512 * u;
        const int row = chunk >> 4, col = chunk & 15;
        *reinterpret_cast<u32x4 *>(buf + row * kWgPitch + 16 * col) = st.c[u];
    }
}

// S^T = K Q^T of one 32-token half of a staged tile for the wavefront's two row
// tiles (K operands read from LDS once, used by both).
__device__ __forceinline__ void wg_qk(const unsigned char *buf, int h, int rr, int g4, const bf16x8 (&qop)[2][4],
                                      f32x4 (&st)[2][2])
{
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int s = 0; s < 2; s++)
            st[a][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; s++) {
        const unsigned char *kr = buf + (32 * h + 16 * s + rr) * kWgPitch + 16 * g4;
        u32x4 kk[4];
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            kk[ks] = *reinterpret_cast<const u32x4 *>(kr + 64 * ks);
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int ks = 0; ks < 4; ks++)
                st[a][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[ks]), qop[a][ks],
                                                                   st[a][s], 0, 0, 0);
    }
}

// O += P V for one 32-token half: the row sums come from a ones column tile; V
// operands of column tile p (d = 16 p + n) come from transposing LDS reads.
// Within a 16-lane group, lane j receives element j % 4 of the 8-byte chunks
// addressed by lanes 4 e + j / 4 (e = 0..3), so lane (rr, g4) addresses token
// 4 g4 + rr / 4 (first read) or 16 + 4 g4 + rr / 4 (second read) at d = 16 p +
// 4 (rr % 4), which yields the lane's 8 tokens in the order of its logits.
__device__ __forceinline__ void wg_pv(const unsigned char *buf, int h, int rr, int g4, const bf16x8 (&aop)[2],
                                      f32x4 (&acc)[2][9])
{
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int a = 0; a < 2; a++)
        acc[a][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[a], ones, acc[a][8], 0, 0, 0);
    const unsigned char *vr = buf + (64 + 32 * h + 4 * g4 + (rr >> 2)) * kWgPitch + 8 * (rr & 3);
#pragma unroll
    for (int p = 0; p < 8; p++) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vr + 32 * p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vr + 16 * kWgPitch + 32 * p));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int a = 0; a < 2; a++)
            acc[a][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[a], bop, acc[a][p], 0, 0, 0);
    }
}

// One staged 64-token tile for the wavefront's two 16-row tiles (this lane: row
// rr of each, 8 logits per 32-token half).  Both QK products come first; the
// reference max m_run is kept on raw logits (the scale is positive) and moves
// lazily, at most once per tile: only when the tile's max exceeds it by more than
// `lazy` (2^8 after scaling), so unnormalised weights stay below 256 and the
// output accumulators are rescaled rarely (a wavefront-uniform branch).  Any
// reference gives the same normalised result.  A lane whose 8 logits of a half
// are all masked gets scale 0 and offset -inf there, so its weights are
// exp2(-inf) = 0 without a select per logit; per-logit masks (a -1e30 sentinel,
// which underflows to 0) are applied only when some lane has a partly live half
// (causal edge, window or sink boundary).  exp2 is the hardware instruction
// (results below 2^-126 flush to zero, which the sum cannot see next to the
// reference term).  Row sums come from the P V product itself (a ones column
// tile), so the accumulators carry them and their rescaling.
__device__ __forceinline__ void wg_tile(const unsigned char *buf, int rr, int g4, const bf16x8 (&qop)[2][4],
                                        const uint32_t (&live)[2][2], bool partial, float scale_log2, float lazy,
                                        float (&m_run)[2], f32x4 (&acc)[2][9])
{
    f32x4 st[2][2][2];                                    // [half][row tile][16-token subtile]
    wg_qk(buf, 0, rr, g4, qop, st[0]);
    wg_qk(buf, 1, rr, g4, qop, st[1]);
    if (partial) {                       // finite sentinel: a dead lane multiplies it by scale 0
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    st[h][a][i >> 2][i & 3] = (live[h][a] >> i) & 1u ? st[h][a][i >> 2][i & 3] : -1e30f;
    }
    float neg[2], m_old[2];
    bool bump[2];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        float mc = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const f32x4 *x = st[h][a];
            const float mh = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                                   fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
            mc = live[h][a] != 0u ? fmaxf(mc, mh) : mc;
        }
        mc = fmaxf(mc, __shfl_xor(mc, 16, kWave));
        mc = fmaxf(mc, __shfl_xor(mc, 32, kWave));
        bump[a] = mc > m_run[a] + lazy;
        m_old[a] = m_run[a];
        m_run[a] = bump[a] ? mc : m_run[a];
        neg[a] = m_run[a] == -INFINITY ? 0.f : -m_run[a] * scale_log2;
    }
    if (__ballot(bump[0] || bump[1])) {
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const float alpha = bump[a] ? __builtin_amdgcn_exp2f(fmaf(m_old[a], scale_log2, neg[a])) : 1.f;
#pragma unroll
            for (int qq = 0; qq < 4; qq++) {
                const float f = __shfl(alpha, 4 * g4 + qq, kWave);
#pragma unroll
                for (int p = 0; p < 9; p++)
                    acc[a][p][qq] *= f;
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
        bf16x8 aop[2];
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const bool lv = live[h][a] != 0u;
            const float s_eff = lv ? scale_log2 : 0.f;
            const float n_eff = lv ? neg[a] : -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; i++)
                aop[a][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(st[h][a][i >> 2][i & 3], s_eff, n_eff));
        }
        wg_pv(buf, h, rr, g4, aop, acc);
    }
}

// The 8 logits of lane group g4 are tokens 4*g4 .. +3 and 16 + 4*g4 .. +3 of the chunk.
__device__ __forceinline__ uint32_t live8(uint32_t m32, int g4)
{
    return ((m32 >> (4 * g4)) & 0xfu) | (((m32 >> (16 + 4 * g4)) & 0xfu) << 4);
}

__global__ __launch_bounds__(512, 1) void attn_wg_kernel(KP P, const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v,
                                                         const int32_t *__restrict__ idx,
                                                         const int32_t *__restrict__ n_idx,
                                                         uint16_t *__restrict__ out, float *__restrict__ lse,
                                                         int n_qtile)
{
    constexpr int D = 128, KS = D / 32;
    __shared__ unsigned long long sh_qm[kWgMaxTiles];      // per tile: queries that selected it
    __shared__ int sh_list[kWgMaxTiles];
    __shared__ unsigned long long sh_lqm[kWgMaxTiles];
    __shared__ __attribute__((aligned(16))) unsigned char sh_kv[2][128 * kWgPitch];
    __shared__ int sh_scan[kWgWaves];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rr = lane & 15, g4 = lane >> 4;
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    const long long per_xcd = (n_items + 7) / 8;
    const long long item = (long long)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= n_items)
        return;
    const int qt = (int)(item % n_qtile);
    const int c = (int)((item / n_qtile) % P.h_kv);
    const int b = (int)(item / ((long long)n_qtile * P.h_kv));
    const Seq s = seq_info(P, b);
    const int QPW = 32 / P.G;                             // queries per wavefront
    const int qwg = kWgWaves * QPW;                       // queries per workgroup (<= 64)
    const int q_lo = qt * qwg;
    const int nq = max(0, min(qwg, s.n_q - q_lo));
    if (nq == 0)                                          // query tile past this sequence's queries
        return;
    const int ntile = (s.n_k + 63) / 64;

    for (int x = tid; x < ntile; x += 512)
        sh_qm[x] = 0ull;
    __syncthreads();
    for (int x = tid; x < nq * P.topk; x += 512) {
        const int qq = x / P.topk, e = x % P.topk;
        const long long qi = s.q_off + q_lo + qq;
        int ns = n_idx[(long long)c * P.rows + qi];
        ns = ns < 0 ? 0 : (ns > P.topk ? P.topk : ns);
        if (e < ns) {
            const int j = idx[((long long)c * P.rows + qi) * P.topk + e];
            if (j >= 0 && j < ntile)
                atomicOr(&sh_qm[j], 1ull << qq);
        }
    }
    __syncthreads();
    // union list: selected blocks, init tiles, window tiles of the workgroup's queries
    const int p_first = s.q0 + q_lo, p_last = s.q0 + q_lo + nq - 1;
    const int init_hi = (min(P.n_init, p_last + 1) + 63) / 64;
    const int win_lo = max(P.n_init, p_first - P.window + 1) / 64, win_hi = p_last / 64;
    const int per = (ntile + 511) / 512;
    int cnt = 0;
    for (int u = 0; u < per; u++) {
        const int j = tid * per + u;
        cnt += (j < ntile && (sh_qm[j] != 0ull || j < init_hi || (j >= win_lo && j <= win_hi))) ? 1 : 0;
    }
    int2 sc = block_scan_int_512(cnt, sh_scan);
    int pos = sc.x;
    for (int u = 0; u < per; u++) {
        const int j = tid * per + u;
        if (j < ntile && (sh_qm[j] != 0ull || j < init_hi || (j >= win_lo && j <= win_hi))) {
            sh_list[pos] = j;
            sh_lqm[pos] = sh_qm[j];
            pos++;
        }
    }
    const int n_list = sc.y;

    // this wavefront's rows: a = 0, 1 -> rows 16a + rr of its 32
    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (s.k_off * P.h_kv + c) * D;
    const uint16_t *vb = v + (s.k_off * P.h_kv + c) * D;
    bf16x8 qop[2][KS];
    int p_row[2], lo_w[2], qbit[2];
    bool row_ok[2];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        const int rq = (16 * a + rr) / P.G;                  // query within the wavefront
        const int ql = w * QPW + rq;                          // query within the workgroup
        row_ok[a] = ql < nq;
        qbit[a] = ql;
        p_row[a] = row_ok[a] ? s.q0 + q_lo + ql : -1;
        lo_w[a] = max(P.n_init, p_row[a] - P.window + 1);
        if (row_ok[a]) {
            const long long qi = s.q_off + q_lo + ql;
            const uint16_t *qp = q + (qi * P.h_q + c * P.G + (16 * a + rr) % P.G) * D + 8 * g4;
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                qop[a][ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                qop[a][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
    }
    // the wavefront's query bits in the 64-bit masks, and its query span for init/window tests
    const int wq_lo = w * QPW, wq_n = max(0, min(QPW, nq - wq_lo));
    const unsigned long long wmask = wq_n > 0 ? (((wq_n == 64) ? ~0ull : ((1ull << wq_n) - 1ull)) << wq_lo) : 0ull;
    const int wp_first = s.q0 + q_lo + wq_lo, wp_last = wp_first + wq_n - 1;
    const int w_init_hi = wq_n > 0 ? (min(P.n_init, wp_last + 1) + 63) / 64 : 0;
    const int w_win_lo = max(P.n_init, wp_first - P.window + 1) / 64, w_win_hi = wq_n > 0 ? wp_last / 64 : -1;

    float m_run[2] = {-INFINITY, -INFINITY};
    const float lazy = 8.f / P.scale_log2;
    f32x4 acc[2][9];                                      // [8]: row sums (ones column tile)
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int p = 0; p < 9; p++)
            acc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Tile t lives in register slot t % kWgStage.  Every iteration: barrier (LDS
    // buffer e&1 holds tile e), compute tile e, write tile e+1 from its slot into
    // the other buffer, then reuse that slot for tile e+1+kWgStage.  Issues and
    // writes are unconditional (clamped to the last tile) so the load counters the
    // compiler tracks are the same on every path.
    // Every query attends at least its own position (window >= 1), so n_list >= 1
    // here; the staging below reads sh_list[0 .. n_list) only.
    WgStage stage[kWgStage];
    const int last = max(n_list - 1, 0);
    if (n_list > 0) {
#pragma unroll
        for (int x = 0; x < kWgStage; x++)
            wg_issue(stage[x], kb, vb, tstride, sh_list[min(x, last)] * 64, s.n_k, tid);
        wg_write(stage[0], sh_kv[0], tid);
        wg_issue(stage[0], kb, vb, tstride, sh_list[min(kWgStage, last)] * 64, s.n_k, tid);
        const int n_iter = ((n_list + kWgStage - 1) / kWgStage) * kWgStage;
        for (int e0 = 0; e0 < n_iter; e0 += kWgStage) {
#pragma unroll
            for (int x = 0; x < kWgStage; x++) {
                const int e = e0 + x;
                __syncthreads();                               // LDS buffer e&1 holds tile e
                const int tile = sh_list[min(e, last)];
                const unsigned long long qm = sh_lqm[min(e, last)];
                const bool need = e < n_list &&
                                  ((qm & wmask) != 0ull || tile < w_init_hi || (tile >= w_win_lo && tile <= w_win_hi));
                if (need) {
                    const unsigned char *buf = sh_kv[e & 1];
                    uint32_t live[2][2];
                    bool any = false, part = false;
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        const int t0 = tile * 64 + 32 * h;
#pragma unroll
                        for (int a = 0; a < 2; a++) {
                            const bool sb = (qm >> qbit[a]) & 1ull;
                            live[h][a] = row_ok[a] ? live8(tile_mask(t0, p_row[a], P.n_init, lo_w[a], sb), g4) : 0u;
                            any = any || live[h][a] != 0u;
                            part = part || (live[h][a] != 0u && live[h][a] != 0xffu);
                        }
                    }
                    if (__ballot(any) != 0ull)
                        wg_tile(buf, rr, g4, qop, live, __ballot(part) != 0ull, P.scale_log2, lazy, m_run, acc);
                }
                const int xn = (x + 1) % kWgStage;
                wg_write(stage[xn], sh_kv[(e + 1) & 1], tid);
                wg_issue(stage[xn], kb, vb, tstride, sh_list[min(e + 1 + kWgStage, last)] * 64, s.n_k, tid);
            }
        }
    }
    // Epilogue: lane (rr, g4) holds d = 16 p + rr of rows 4 g4 + r4; normalised bf16
    // rows are transposed through this wavefront's 32-row slice of the (now
    // idle) staging buffers and stored as 16-byte row pieces.
    __syncthreads();
    unsigned char *ob = &sh_kv[0][0] + w * 32 * kWgPitch;
#pragma unroll
    for (int a = 0; a < 2; a++) {
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
            const int row = 4 * g4 + r4;                      // row within the 16-row tile a
            const float lrow = acc[a][8][r4];                 // sum of the bf16 weights of the row
            const float inv = 1.0f / lrow;
            uint16_t *orow = reinterpret_cast<uint16_t *>(ob + (16 * a + row) * kWgPitch);
#pragma unroll
            for (int p = 0; p < 8; p++)
                orow[16 * p + rr] = f32_to_bf16(acc[a][p][r4] * inv);
            const float mrow = __shfl(m_run[a], row, kWave);
            const int ql = w * QPW + (16 * a + row) / P.G;
            if (lse && rr == 0 && ql < nq) {
                const long long oq = s.q_off + q_lo + ql;
                const int h = c * P.G + (16 * a + row) % P.G;
                lse[(long long)h * P.total_q + oq] = (mrow * P.scale_log2 + log2f(lrow)) * 0.69314718055994531f;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                   // lgkmcnt(0): this wavefront's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 8; t++) {
        const int u = lane + 64 * t;                       // 512 pieces: 32 rows x 16
        const int row = u >> 4, piece = u & 15;
        const int ql = w * QPW + row / P.G;
        if (ql < nq) {
            const long long oq = s.q_off + q_lo + ql;
            const int h = c * P.G + row % P.G;
            *reinterpret_cast<u32x4 *>(out + (oq * P.h_q + h) * D + 8 * piece) =
                *reinterpret_cast<const u32x4 *>(ob + row * kWgPitch + 16 * piece);
        }
    }
}

bool wg_fwd_ok(const KP &P, int dtype)
{
    return dtype == 1 && !P.shared && P.d == 128 && P.g == 64 && (P.G == 4 || P.G == 8 || P.G == 16) &&
           P.max_k <= kWgMaxTiles * 64 && P.max_q >= 256 && !getenv("SPARSE_ATTN_NO_WG");
}

hipError_t launch_fwd_wg(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                         const int32_t *n_idx, void *out, float *lse, void *ev0, void *ev1, hipStream_t st)
{
    const int qwg = kWgWaves * (32 / P.G);
    const int n_qtile = (P.max_q + qwg - 1) / qwg;
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    const long long grid = ((n_items + 7) / 8) * 8;
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    attn_wg_kernel<<<dim3((unsigned)grid), dim3(512), 0, st>>>(P, (const uint16_t *)q, (const uint16_t *)k,
                                                               (const uint16_t *)v, idx, n_idx, (uint16_t *)out,
                                                               lse, n_qtile);
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev1, st);
    return hipGetLastError();
}

bool tile_fwd_ok(const KP &P, int dtype)
{
    return dtype == 1 && !P.shared && P.G >= 4 && P.G <= 16 && 16 % P.G == 0 && P.g % 32 == 0 &&
           P.max_k <= kTileMax * 32 && P.max_q > 64;
}

hipError_t launch_fwd_tile(const KP &P, const void *q, const void *k, const void *v, const int32_t *idx,
                           const int32_t *n_idx, void *out, float *lse, void *ev0, void *ev1, hipStream_t st)
{
    const int qpw = 16 / P.G;
    const int n_qtile = (P.max_q + kTileWaves * qpw - 1) / (kTileWaves * qpw);
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    const long long grid = ((n_items + 7) / 8) * 8;
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    if (P.d == 128)
        attn_tile_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, st>>>(
            P, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
            n_qtile);
    else
        attn_tile_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, st>>>(
            P, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
            n_qtile);
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev1, st);
    return hipGetLastError();
}

bool mfma_fwd_ok(const KP &P, int dtype)
{
    if (dtype != 1)
        return false;
    long long rows = P.shared ? (long long)P.max_q * P.G : P.G;
    return rows <= 16;
}

int mfma_fwd_splits(const KP &P)
{
    long long a_max = (long long)P.n_init + (long long)P.topk * P.g + P.window + (P.shared ? P.max_q : 0);
    if (a_max > P.max_k)
        a_max = P.max_k;
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
    if (sp > 64)
        sp = 64;
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
