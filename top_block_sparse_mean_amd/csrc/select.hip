// select.hip -- top-k block selection on gfx950.
//
// Score of candidate block j for a selection row and KV head c: the row's
// query heads of group c (and, for a shared row, all its queries) summed into
// one fp32 selector query Qs, dotted with the fp32 pooled key K~_j (SparDA
// summary, Method: one selector head per GQA group; LSA deep-read, §2.3-§2.4).
// Ranking uses the raw dot: the positive 1/sqrt(d) factor cannot change the
// order, and leaving it out avoids a rounding step that could merge two
// neighbouring fp32 scores.  Equal scores keep the lower index.
//
// Kernels:
//   score_rows    decode / shared rows: 64 candidates per workgroup, one round of
//                 16 B loads per lane (wavefront dot products, xor-shuffle sums),
//                 order keys to the workspace.
//   score_tile    prefill: 64 rows x 64 blocks per workgroup, operands staged in
//                 LDS, fp32 MFMA 16x16x4 (fp32-accurate products), writes keys.
//   topk_wave     one wavefront per row, keys in registers (<= 2048 candidates).
//   topk_block    one workgroup per row, 8-bit radix select over the workspace.
//
// Top-k rule on the keys: the k-th largest key tau is found by a binary search
// on its bits (wavefront) or by 8-bit radix passes (workgroup); the output is
// every key > tau plus the lowest-index keys == tau needed to reach k, written
// in ascending index order by ballot compaction.
#include <stdlib.h>

#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- row geometry

struct RowGeo {
    int b, n_k, p_sel;
    long long q_first, q_last;   // packed query range summed into the selector
    int j_lo, j_hi, n_cand, need;
    long long k_off;
};

__device__ __forceinline__ RowGeo row_geo(const KP &P, long long row)
{
    RowGeo r;
    if (P.shared) {
        r.b = (int)row;
        Seq s = seq_info(P, r.b);
        r.q_first = s.q_off;
        r.q_last = s.q_off + s.n_q;
        r.p_sel = s.q0 - 1;
        r.n_k = s.n_k;
        r.k_off = s.k_off;
    } else {
        r.b = seq_of_query(P, row);
        Seq s = seq_info(P, r.b);
        r.q_first = row;
        r.q_last = row + 1;
        r.p_sel = s.q0 + (int)(row - s.q_off);
        r.n_k = s.n_k;
        r.k_off = s.k_off;
    }
    cand_range(P.g, P.n_init, P.window, r.n_k, r.p_sel, r.j_lo, r.j_hi);
    const int cap = P.g == 1 ? P.max_k : P.nb_max;     // rows of the key table / workspace
    r.j_hi = min(r.j_hi, cap);
    r.j_lo = min(r.j_lo, r.j_hi);
    r.n_cand = r.j_hi - r.j_lo;
    int k = P.topk_per_seq ? P.topk_per_seq[r.b] : P.topk;
    k = k < 0 ? 0 : (k > P.topk ? P.topk : k);
    r.need = k < r.n_cand ? k : r.n_cand;
    return r;
}

// Write idx = j_lo .. j_hi-1 (all candidates kept) and the -1 padding.
__device__ __forceinline__ void write_all(const KP &P, int32_t *out, const RowGeo &r, int t, int nt)
{
    for (int s = t; s < P.topk; s += nt)
        out[s] = s < r.n_cand ? r.j_lo + s : -1;
}

// ---------------------------------------------------------------- top-k cores

// One wavefront: the `need` largest of n keys (key i at lane i % 64, slot i / 64),
// indices j_base + i written ascending to out[0 .. need).
template <int KPL>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[KPL], int n, int need, int j_base, int32_t *out)
{
    const int lane = lane_id();
    // counts come from ballots (one scalar popcount per slot): no cross-lane data moves
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < KPL; m++)
            cnt += __popcll(__ballot(m * kWave + lane < n && key[m] >= cand));
        if (cnt >= need)
            tau = cand;
    }
    int gt = 0;
#pragma unroll
    for (int m = 0; m < KPL; m++)
        gt += __popcll(__ballot(m * kWave + lane < n && key[m] > tau));
    int need_eq = need - gt;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        int i = m * kWave + lane;
        bool valid = i < n;
        bool is_gt = valid && key[m] > tau;
        bool is_eq = valid && key[m] == tau;
        unsigned long long meq = __ballot(is_eq);
        int rank = eq_seen + lanes_below(meq);
        eq_seen += __popcll(meq);
        bool s = is_gt || (is_eq && rank < need_eq);
        unsigned long long ms = __ballot(s);
        if (s)
            out[base + lanes_below(ms)] = j_base + i;
        base += __popcll(ms);
    }
}

template <int NT>
__device__ __forceinline__ int2 block_scan_flag(bool f, int *sh)
{
    unsigned long long m = __ballot(f);
    int w = threadIdx.x / kWave;
    if (lane_id() == 0)
        sh[w] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) {
        int c = sh[i];
        off += i < w ? c : 0;
        tot += c;
    }
    __syncthreads();
    return make_int2(off + lanes_below(m), tot);
}

// One workgroup: the `need` largest of keys[0 .. n) (global memory), 8-bit radix.
template <int NT>
__device__ void block_topk(const uint32_t *__restrict__ keys, int n, int need, int j_base, int32_t *out)
{
    __shared__ int hist[256];
    __shared__ int sh_scan[NT / kWave];
    __shared__ int sh_digit, sh_above;
    const int tid = threadIdx.x, lane = lane_id();
    uint32_t prefix = 0, pmask = 0;
    int rem = need;
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += NT)
            hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            uint32_t k = keys[i];
            if ((k & pmask) == prefix)
                atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < kWave) {
            int c[4], s = 0;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                c[q] = hist[255 - 4 * lane - q];
                s += c[q];
            }
            int incl = s;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                int t = __shfl_up(incl, o, kWave);
                if (lane >= o)
                    incl += t;
            }
            unsigned long long mk = __ballot(incl >= rem);
            int first = __ffsll((long long)mk) - 1;
            if (lane == first) {
                int run = incl - s;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if (run + c[q] >= rem) {
                        sh_digit = 255 - 4 * lane - q;
                        sh_above = run;
                        break;
                    }
                    run += c[q];
                }
            }
        }
        __syncthreads();
        prefix |= ((uint32_t)sh_digit) << shift;
        pmask |= 255u << shift;
        rem -= sh_above;
        __syncthreads();
    }
    const uint32_t tau = prefix;
    const int need_eq = rem;
    int sel_base = 0, eq_seen = 0;
    for (int base = 0; base < n; base += NT) {
        int i = base + tid;
        bool valid = i < n;
        uint32_t k = valid ? keys[i] : 0u;
        bool is_gt = valid && k > tau, is_eq = valid && k == tau;
        int2 e = block_scan_flag<NT>(is_eq, sh_scan);
        int rank = eq_seen + e.x;
        eq_seen += e.y;
        bool s = is_gt || (is_eq && rank < need_eq);
        int2 p = block_scan_flag<NT>(s, sh_scan);
        if (s)
            out[sel_base + p.x] = j_base + i;
        sel_base += p.y;
    }
}

// ---------------------------------------------------------------- scoring helpers

// Lanes per key row and elements per lane for 16 B loads: pooled fp32 keys
// (4 floats per lane) or raw keys at g = 1 (8 bf16, or 4 fp32, per lane).
template <typename KT, int D>
struct RowDot {
    static constexpr int VPL = 16 / sizeof(KT) < 8 ? 16 / sizeof(KT) : 8, L = D / VPL;
};

// Pointer to key row j of (sequence, KV head c) for scoring: pooled fp32 or raw.
template <typename KT, int D>
__device__ __forceinline__ const KT *key_row(const KP &P, const KT *base, const RowGeo &r, int c, int j)
{
    if (P.g == 1)
        return base + ((r.k_off + j) * P.h_kv + c) * D;
    return base + (((long long)c * P.batch + r.b) * P.nb_max + j) * D;
}

// ---------------------------------------------------------------- score_rows (split)

// Selector slice of this lane: Qs[sub*VPL .. +VPL] summed over the row's queries and group c's heads.
template <typename T, int D, int VPL>
__device__ __forceinline__ void selector_slice(const KP &P, const T *q, const RowGeo &r, int c, int sub,
                                               float (&qs)[VPL])
{
#pragma unroll
    for (int e = 0; e < VPL; e++)
        qs[e] = 0.f;
    for (long long i = r.q_first; i < r.q_last; i++) {
        const T *qi = q + (i * P.h_q + (long long)c * P.G) * D + sub * VPL;
        for (int h = 0; h < P.G; h++) {
#pragma unroll
            for (int e = 0; e < VPL; e++) {
                if constexpr (sizeof(T) == 2)
                    qs[e] += bf16_to_f32(qi[h * D + e]);
                else
                    qs[e] += qi[h * D + e];
            }
        }
    }
}

// Partial dot of one 16 B key slice with this lane's selector slice.
template <int VPL>
__device__ __forceinline__ float slice_dot(const uint4 &raw, const float (&qv)[VPL])
{
    if constexpr (VPL == 4) {
        return qv[0] * __uint_as_float(raw.x) + qv[1] * __uint_as_float(raw.y) + qv[2] * __uint_as_float(raw.z) +
               qv[3] * __uint_as_float(raw.w);
    } else {
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++)
            part += qv[2 * e] * __uint_as_float(wd[e] << 16) + qv[2 * e + 1] * __uint_as_float(wd[e] & 0xffff0000u);
        return part;
    }
}

// grid: (rows * n_chunk, h_kv), CH candidates per workgroup in rounds of U x NG rows;
// writes order keys to ws[(c*rows+row)*stride + j].  The loads of round r+1 are
// issued before round r is reduced; the selector slice is built while the first
// round is in flight.
template <typename T, typename KT, int D, int CH>
__global__ __launch_bounds__(256) void score_rows_kernel(KP P, const T *__restrict__ q,
                                                         const KT *__restrict__ kbase,
                                                         uint32_t *__restrict__ ws, long long stride, int n_chunk)
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 4 * GPW;
    constexpr int U = 64 / NG < 1 ? 1 : 64 / NG;      // 64 rows per round
    constexpr int RW = U * NG;
    const long long row = blockIdx.x / n_chunk;
    const int chunk = (int)(blockIdx.x % n_chunk);
    const int c = blockIdx.y;
    RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand)
        return;
    const int j0 = r.j_lo + chunk * CH;
    const int j1 = min(j0 + CH, r.j_hi);
    if (j0 >= j1)
        return;
    const int tid = threadIdx.x, lane = lane_id(), sub = lane % L, grp = (tid / kWave) * GPW + lane / L;
    const int rounds = (j1 - j0 + RW - 1) / RW;
    uint4 ra[U], rb[U];
    auto load = [&](uint4 (&raw)[U], int rd) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            int j = min(j0 + rd * RW + u * NG + grp, j1 - 1);
            raw[u] = reinterpret_cast<const uint4 *>(key_row<KT, D>(P, kbase, r, c, j))[sub];
        }
    };
    uint32_t *dst = ws + ((long long)c * P.rows + row) * stride;
    float qv[VPL];
    auto reduce = [&](const uint4 (&raw)[U], int rd) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            float sc = group_sum<L>(slice_dot<VPL>(raw[u], qv));
            int j = j0 + rd * RW + u * NG + grp;
            if (sub == 0 && j < j1)
                dst[j] = order_key(sc);
        }
    };
    load(ra, 0);
    selector_slice<T, D, VPL>(P, q, r, c, sub, qv);
    for (int rd = 0; rd < rounds; rd += 2) {
        if (rd + 1 < rounds)
            load(rb, rd + 1);
        reduce(ra, rd);
        if (rd + 1 >= rounds)
            break;
        if (rd + 2 < rounds)
            load(ra, rd + 2);
        reduce(rb, rd + 1);
    }
}

// ---------------------------------------------------------------- select_row (fused)

// One 1024-thread workgroup per (row, KV head) for rows with at most 64*KPL
// candidates: every lane issues the loads of all its key rows at once, the
// order keys go to LDS, wavefront 0 selects.  No workspace, one launch.
template <typename T, typename KT, int D, int KPL>
__global__ __launch_bounds__(1024) void select_row_kernel(KP P, const T *__restrict__ q,
                                                          const KT *__restrict__ kbase,
                                                          int32_t *__restrict__ idx, int32_t *__restrict__ n_idx)
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 16 * GPW, MAXC = 64 * KPL;
    constexpr int U = (MAXC + NG - 1) / NG;
    __shared__ uint32_t keys[MAXC];
    const long long row = blockIdx.x;
    const int c = blockIdx.y;
    const int tid = threadIdx.x, lane = lane_id(), sub = lane % L, grp = (tid / kWave) * GPW + lane / L;
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (tid == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, tid, 1024);
        return;
    }
    const int n = min(r.n_cand, MAXC);
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        int jj = min(u * NG + grp, n - 1);
        raw[u] = reinterpret_cast<const uint4 *>(key_row<KT, D>(P, kbase, r, c, r.j_lo + jj))[sub];
    }
    float qv[VPL];
    selector_slice<T, D, VPL>(P, q, r, c, sub, qv);
#pragma unroll
    for (int u = 0; u < U; u++) {
        float sc = group_sum<L>(slice_dot<VPL>(raw[u], qv));
        int jj = u * NG + grp;
        if (sub == 0 && jj < n)
            keys[jj] = order_key(sc);
    }
    __syncthreads();
    if (tid < kWave) {
        uint32_t kr[KPL];
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            int i = m * kWave + lane;
            kr[m] = i < n ? keys[i] : 0u;
        }
        wave_topk<KPL>(kr, n, min(r.need, n), r.j_lo, out);
        for (int s2 = r.need + lane; s2 < P.topk; s2 += kWave)
            out[s2] = -1;
    }
}

// ---------------------------------------------------------------- score_tile (MFMA fp32)

// Prefill rows (one per query).  grid: (block chunks of 64, row tiles of 64, h_kv * batch).
// 4 wavefronts in a 2 x 2 arrangement, each a 32 x 32 tile of 2 x 2 MFMA 16x16x4 f32.
// MFMA 16x16x4 f32 operands: lane l gives A[l%16][l/16] and B[l/16][l%16];
// the result lane l holds D[4*(l/16)+i][l%16], i = 0..3.
template <typename T, typename KT, int D>
__global__ __launch_bounds__(256) void score_tile_kernel(KP P, const T *__restrict__ q,
                                                         const KT *__restrict__ kbase,
                                                         uint32_t *__restrict__ ws, long long stride)
{
    constexpr int TR = 64, TJ = 64, LD = D + 4;
    __shared__ float qs_sh[TR * LD];
    __shared__ float kt_sh[TJ * LD];
    const int b = blockIdx.z % P.batch, c = blockIdx.z / P.batch;
    Seq s = seq_info(P, b);
    const int r0 = blockIdx.y * TR;
    if (r0 >= s.n_q)
        return;
    const int r_end = min(r0 + TR, s.n_q);
    // candidate range of the tile's last row bounds every row of the tile
    int jlo_last, jhi_last;
    cand_range(P.g, P.n_init, P.window, s.n_k, s.q0 + r_end - 1, jlo_last, jhi_last);
    jhi_last = min(jhi_last, (int)stride);
    const int j0 = jlo_last + blockIdx.x * TJ;
    if (j0 >= jhi_last)
        return;
    const int tid = threadIdx.x;
    // stage Qs: 64 rows x D, 8 elements per item
    for (int it = tid; it < TR * (D / 8); it += 256) {
        int rr = it / (D / 8), e0 = (it % (D / 8)) * 8;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r0 + rr < r_end) {
            long long i = s.q_off + r0 + rr;
            for (int h = 0; h < P.G; h++) {
                float x[8];
                load8(q + (i * P.h_q + (long long)c * P.G + h) * D + e0, x);
#pragma unroll
                for (int e = 0; e < 8; e++)
                    acc[e] += x[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            qs_sh[rr * LD + e0 + e] = acc[e];
    }
    // stage keys: 64 candidate rows x D
    for (int it = tid; it < TJ * (D / 8); it += 256) {
        int jj = it / (D / 8), e0 = (it % (D / 8)) * 8;
        int j = j0 + jj;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (j < jhi_last) {
            if (P.g == 1)
                load8(kbase + ((s.k_off + j) * P.h_kv + c) * D + e0, x);
            else
                load8(kbase + (((long long)c * P.batch + b) * P.nb_max + j) * D + e0, x);
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            kt_sh[jj * LD + e0 + e] = x[e];
    }
    __syncthreads();
    const int lane = lane_id(), w = tid / kWave;
    const int wr = (w >> 1) * 32, wj = (w & 1) * 32;
    floatx4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int bb = 0; bb < 2; bb++)
            acc[a][bb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int li = lane % 16, lk = lane / 16;
#pragma unroll 8
    for (int e = 0; e < D; e += 4) {
        float av[2], bv[2];
#pragma unroll
        for (int a = 0; a < 2; a++)
            av[a] = qs_sh[(wr + a * 16 + li) * LD + e + lk];
#pragma unroll
        for (int bb = 0; bb < 2; bb++)
            bv[bb] = kt_sh[(wj + bb * 16 + li) * LD + e + lk];
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int bb = 0; bb < 2; bb++)
                acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[bb], acc[a][bb], 0, 0, 0);
    }
    // epilogue: row = r0 + wr + a*16 + 4*lk + i, block = j0 + wj + bb*16 + li
#pragma unroll
    for (int a = 0; a < 2; a++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int rl = r0 + wr + a * 16 + 4 * lk + i;
            if (rl >= r_end)
                continue;
            int jl, jh;
            cand_range(P.g, P.n_init, P.window, s.n_k, s.q0 + rl, jl, jh);
            jh = min(jh, (int)stride);
            uint32_t *dst = ws + ((long long)c * P.rows + s.q_off + rl) * stride;
#pragma unroll
            for (int bb = 0; bb < 2; bb++) {
                int j = j0 + wj + bb * 16 + li;
                if (j >= jl && j < jh)
                    dst[j] = order_key(acc[a][bb][i]);
            }
        }
    }
}

// ---------------------------------------------------------------- top-k over the workspace

// 4 wavefronts per workgroup, one row each (<= 64 * KPL candidates).  grid: (ceil(rows/4), h_kv).
template <int KPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(KP P, const uint32_t *__restrict__ ws,
                                                        long long stride, int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ n_idx)
{
    const long long row = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    const int c = blockIdx.y, lane = lane_id();
    if (row >= P.rows)
        return;
    // the candidate range of any row with candidates starts at n_init / g: load first, then
    // resolve the row's geometry while the loads are in flight
    const int j_first = P.n_init / P.g;
    const uint32_t *src = ws + ((long long)c * P.rows + row) * stride;
    uint32_t kr[KPL];
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        long long j = j_first + m * kWave + lane;
        kr[m] = j < stride ? src[j] : 0u;
    }
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (lane == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, lane, kWave);
        return;
    }
    wave_topk<KPL>(kr, r.n_cand, r.need, r.j_lo, out);
    for (int s = r.need + lane; s < P.topk; s += kWave)
        out[s] = -1;
}

// One 1024-thread workgroup per row with up to 1024 * KPT candidates held in
// registers (key i in thread i % 1024, slot i / 1024).  tau is found by a
// binary search on its bits; counts are wave ballots summed through LDS (one
// barrier per bit).  The output is written in index order from per-(slot, wave)
// counts, so it needs only three more barriers.  grid: (rows, h_kv).
template <int KPT>
__global__ __launch_bounds__(1024) void topk_regs_kernel(KP P, const uint32_t *__restrict__ ws, long long stride,
                                                         int32_t *__restrict__ idx, int32_t *__restrict__ n_idx)
{
    constexpr int NT = 1024, NW = NT / kWave;
    __shared__ int sh_cnt[2][NW];
    __shared__ int sh_gt[KPT][NW], sh_eq[KPT][NW];
    const long long row = blockIdx.x;
    const int c = blockIdx.y, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int j_first = P.n_init / P.g;
    const uint32_t *src = ws + ((long long)c * P.rows + row) * stride;
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (tid == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, tid, NT);
        return;
    }
    const int n = min(r.n_cand, NT * KPT);
    const int need = min(r.need, n);
    const int slots = (n + NT - 1) / NT;            // slots holding candidates (uniform)
    uint32_t kr[KPT];
#pragma unroll
    for (int m = 0; m < KPT; m++) {
        long long j = j_first + (long long)m * NT + tid;
        kr[m] = (m < slots && j < stride) ? src[j] : 0u;
    }
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < KPT; m++)
            if (m < slots)
                cnt += __popcll(__ballot(m * NT + tid < n && kr[m] >= cand));
        if (lane == 0)
            sh_cnt[bit & 1][w] = cnt;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int x = 0; x < NW; x++)
            tot += sh_cnt[bit & 1][x];
        if (tot >= need)
            tau = cand;
    }
    // per (slot, wave) counts of keys above tau and equal to tau
    int g_tot = 0;
#pragma unroll
    for (int m = 0; m < KPT; m++) {
        if (m >= slots)
            break;
        bool valid = m * NT + tid < n;
        int g = __popcll(__ballot(valid && kr[m] > tau));
        int e = __popcll(__ballot(valid && kr[m] == tau));
        g_tot += g;
        if (lane == 0) {
            sh_gt[m][w] = g;
            sh_eq[m][w] = e;
        }
    }
    __syncthreads();                                   // every wave has read sh_cnt too
    if (lane == 0)
        sh_cnt[0][w] = g_tot;
    __syncthreads();
    int n_gt = 0;
#pragma unroll
    for (int x = 0; x < NW; x++)
        n_gt += sh_cnt[0][x];
    const int need_eq = need - n_gt;
    // output position of a selected key = selected keys before it in index order
    // (index = slot * 1024 + wave * 64 + lane)
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int m = 0; m < KPT; m++) {
        if (m >= slots)
            break;
        int eq_m_before_w = 0, gt_m_before_w = 0, eq_m = 0, gt_m = 0;
#pragma unroll
        for (int x = 0; x < NW; x++) {
            int e = sh_eq[m][x], g = sh_gt[m][x];
            eq_m_before_w += x < w ? e : 0;
            gt_m_before_w += x < w ? g : 0;
            eq_m += e;
            gt_m += g;
        }
        const bool valid = m * NT + tid < n;
        const bool is_gt = valid && kr[m] > tau, is_eq = valid && kr[m] == tau;
        const unsigned long long meq = __ballot(is_eq);
        const int eq_rank = eq_before + eq_m_before_w + lanes_below(meq);
        const bool s_eq = is_eq && eq_rank < need_eq;
        const unsigned long long msel = __ballot(is_gt || s_eq);
        // selected before this lane = gt before + eq selected before
        const int eq_sel_before_wave = min(max(need_eq - eq_before, 0), eq_m_before_w);
        const int pos = sel_before + gt_m_before_w + eq_sel_before_wave + lanes_below(msel);
        if (is_gt || s_eq)
            out[pos] = r.j_lo + m * NT + tid;
        sel_before += gt_m + min(max(need_eq - eq_before, 0), eq_m);
        eq_before += eq_m;
    }
    for (int s2 = need + tid; s2 < P.topk; s2 += NT)
        out[s2] = -1;
}

// One workgroup per row.  grid: (rows, h_kv).
template <int NT>
__global__ __launch_bounds__(NT) void topk_block_kernel(KP P, const uint32_t *__restrict__ ws,
                                                        long long stride, int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ n_idx)
{
    const long long row = blockIdx.x;
    const int c = blockIdx.y;
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (threadIdx.x == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, threadIdx.x, NT);
        return;
    }
    block_topk<NT>(ws + ((long long)c * P.rows + row) * stride + r.j_lo, r.n_cand, r.need, r.j_lo, out);
    for (int s = r.need + (int)threadIdx.x; s < P.topk; s += NT)
        out[s] = -1;
}

// Every row: n_idx = 0 and no index (k = 0 everywhere).
__global__ void select_empty_kernel(KP P, int32_t *__restrict__ n_idx)
{
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < P.rows * P.h_kv)
        n_idx[i] = 0;
}

// ---------------------------------------------------------------- dispatch

static constexpr int kWaveTopkMax = 2048;
static constexpr int kRowMaxCand = 1024;
static constexpr int kSplitChunk = 512;  // candidates per scoring workgroup (8 rounds of 64)

size_t select_workspace_bytes(const KP &P, int plan)
{
    if (plan == kSelectEmpty || plan == kSelectRow)
        return 0;
    long long stride = P.g == 1 ? P.max_k : P.nb_max;
    return (size_t)P.h_kv * (size_t)P.rows * (size_t)stride * sizeof(uint32_t);
}

int select_plan(const KP &P)
{
    if (P.topk == 0)
        return kSelectEmpty;
    bool few_rows = P.shared || P.max_q <= 8;
    long long max_cand = P.g == 1 ? P.max_k : P.nb_max;
    int plan = !few_rows ? kSelectTile : (max_cand <= kRowMaxCand ? kSelectRow : kSelectSplit);
    if (const char *e = getenv("SPARSE_ATTN_SELECT_PLAN")) {       // tuning override
        int v = atoi(e);
        if (few_rows && (v == kSelectSplit || (v == kSelectRow && max_cand <= kRowMaxCand)))
            plan = v;
    }
    return plan;
}

template <typename T, int D>
static hipError_t launch_select_t(const KP &P, const void *q_sel, const float *k_cmp, const void *k,
                                  int32_t *idx, int32_t *n_idx, void *ws, hipStream_t st)
{
    const T *q = (const T *)q_sel;
    int plan = select_plan(P);
    long long stride = P.g == 1 ? P.max_k : P.nb_max;
    uint32_t *wsk = (uint32_t *)ws;
    if (plan == kSelectEmpty) {
        long long n = P.rows * P.h_kv;
        select_empty_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(P, n_idx);
        return hipGetLastError();
    }
    if (plan == kSelectRow) {
        dim3 grid((unsigned)P.rows, (unsigned)P.h_kv);
        if (P.g == 1) {
            if (stride <= 512)
                select_row_kernel<T, T, D, 8><<<grid, dim3(1024), 0, st>>>(P, q, (const T *)k, idx, n_idx);
            else
                select_row_kernel<T, T, D, 16><<<grid, dim3(1024), 0, st>>>(P, q, (const T *)k, idx, n_idx);
        } else {
            if (stride <= 512)
                select_row_kernel<T, float, D, 8><<<grid, dim3(1024), 0, st>>>(P, q, k_cmp, idx, n_idx);
            else
                select_row_kernel<T, float, D, 16><<<grid, dim3(1024), 0, st>>>(P, q, k_cmp, idx, n_idx);
        }
        return hipGetLastError();
    }
    if (plan == kSelectSplit) {
        int n_chunk = (int)((stride + kSplitChunk - 1) / kSplitChunk);
        dim3 grid((unsigned)(P.rows * n_chunk), (unsigned)P.h_kv);
        if (P.g == 1)
            score_rows_kernel<T, T, D, kSplitChunk><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride,
                                                                              n_chunk);
        else
            score_rows_kernel<T, float, D, kSplitChunk><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, stride,
                                                                                  n_chunk);
    } else {
        dim3 grid((unsigned)((stride + 63) / 64), (unsigned)((P.max_q + 63) / 64), (unsigned)(P.h_kv * P.batch));
        if (P.g == 1)
            score_tile_kernel<T, T, D><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride);
        else
            score_tile_kernel<T, float, D><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, stride);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    dim3 tgrid((unsigned)((P.rows + 3) / 4), (unsigned)P.h_kv);
    if (stride <= 256)
        topk_wave_kernel<4><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (stride <= 512)
        topk_wave_kernel<8><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (stride <= 1024)
        topk_wave_kernel<16><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (stride <= kWaveTopkMax)
        topk_wave_kernel<32><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (stride <= 8192)
        topk_regs_kernel<8><<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(1024), 0, st>>>(P, wsk, stride, idx,
                                                                                           n_idx);
    else if (stride <= 32768)
        topk_regs_kernel<32><<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(1024), 0, st>>>(P, wsk, stride, idx,
                                                                                            n_idx);
    else
        topk_block_kernel<1024><<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(1024), 0, st>>>(
            P, wsk, stride, idx, n_idx);
    return hipGetLastError();
}

hipError_t launch_select(const KP &P, int dtype, const void *q_sel, const float *k_cmp, const void *k,
                         int32_t *idx, int32_t *n_idx, void *ws, hipStream_t st)
{
    if (dtype == 1)
        return P.d == 128 ? launch_select_t<uint16_t, 128>(P, q_sel, k_cmp, k, idx, n_idx, ws, st)
                          : launch_select_t<uint16_t, 64>(P, q_sel, k_cmp, k, idx, n_idx, ws, st);
    return P.d == 128 ? launch_select_t<float, 128>(P, q_sel, k_cmp, k, idx, n_idx, ws, st)
                      : launch_select_t<float, 64>(P, q_sel, k_cmp, k, idx, n_idx, ws, st);
}

} // namespace sa
