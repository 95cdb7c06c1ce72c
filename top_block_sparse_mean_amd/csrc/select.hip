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

#include <algorithm>

#include "append_common.hpp"
#include "mfma_common.hpp"
#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

// Score-key rows (the workspace of the scoring plans) store candidate j of a row at
// column j + key_col0(P), in rows whose pitch is a multiple of 32: the first
// candidate's group of 32 starts a 128-byte line, so the tile scorer's 32-candidate
// runs are whole cache lines.
__host__ __device__ __forceinline__ int key_col0(const KP &P) { return (32 - first_cand(P) % 32) % 32; }

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
    row_cands(P, r.n_k, r.p_sel, r.j_lo, r.j_hi);
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

// One wavefront, given tau = the need-th largest of n keys (or any threshold with
// exactly need keys at or above it; key i at lane i % 64, slot i / 64): emit(slot, i)
// for every key above tau and the lowest-index keys equal to it, need in all, slots
// 0 .. need-1 in ascending i.
template <int KPL, typename Emit>
__device__ __forceinline__ void emit_above(const uint32_t (&key)[KPL], int n, int need, uint32_t tau, Emit emit)
{
    const int lane = lane_id();
    int gt = 0;
#pragma unroll
    for (int m = 0; m < KPL; m++)
        gt += __popcll(__ballot(m * kWave + lane < n && key[m] > tau));
    const int need_eq = need - gt;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int i = m * kWave + lane;
        const bool valid = i < n;
        const bool is_gt = valid && key[m] > tau;
        const bool is_eq = valid && key[m] == tau;
        const unsigned long long meq = __ballot(is_eq);
        const int rank = eq_seen + lanes_below(meq);
        eq_seen += __popcll(meq);
        const bool s = is_gt || (is_eq && rank < need_eq);
        const unsigned long long ms = __ballot(s);
        const int slot = base + lanes_below(ms);
        if (s && slot < need)
            emit(slot, i);
        base += __popcll(ms);
    }
}

// One wavefront: the `need` largest of n keys (key i at lane i % 64, slot i / 64);
// emit(slot, i) is called for each selected key, slots 0 .. need-1 in ascending i.
template <int KPL, typename Emit>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[KPL], int n, int need, Emit emit)
{
    const int lane = lane_id();
    // counts come from ballots (one scalar popcount per slot): no cross-lane data moves.
    // A threshold with exactly `need` keys at or above it ends the search: those keys
    // are the selection (keys equal to it included), whatever the lower bits.
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < KPL; m++)
            cnt += __popcll(__ballot(m * kWave + lane < n && key[m] >= cand));
        if (cnt >= need)
            tau = cand;
        if (cnt == need)
            break;
    }
    emit_above<KPL>(key, n, need, tau, emit);
}

// Writes the selected block indices j_base + i to out[slot].
struct EmitIdx {
    int32_t *out;
    int j_base;
    __device__ void operator()(int slot, int i) const { out[slot] = j_base + i; }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = min(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

// ---------------------------------------------------------------- boundary scores

// The selection audit (P.boundary): per (row, KV head) the need-th largest score (the
// smallest one kept) and the (need+1)-th (the largest one left out), from the very
// keys the selection ranked.  Rows that keep every candidate or none have neither.
__device__ __forceinline__ void boundary_none(const KP &P, long long row, int c)
{
    float *dst = P.boundary + (((long long)c * P.rows + row) << 1);
    dst[0] = __builtin_nanf("");
    dst[1] = __builtin_nanf("");
}

__device__ __forceinline__ void boundary_store(const KP &P, long long row, int c, uint32_t k_kept, uint32_t k_left)
{
    float *dst = P.boundary + (((long long)c * P.rows + row) << 1);
    dst[0] = key_value(k_kept) * P.boundary_scale;
    dst[1] = key_value(k_left) * P.boundary_scale;
}

// Marks key i as selected in a bit set in LDS (any lane may mark any key).
__device__ __forceinline__ void mark_selected(uint32_t *bits, int i) { atomicOr(&bits[i >> 5], 1u << (i & 31)); }

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wavefront holding a row's n keys (key i at lane i % 64, slot i / 64), the
// selected ones marked in `bits`: stores the smallest selected and the largest
// unselected key (0 < need < n, so both exist).
template <int KPL>
__device__ __forceinline__ void wave_boundary(const KP &P, long long row, int c, const uint32_t (&key)[KPL], int n,
                                              const uint32_t *bits)
{
    const int lane = lane_id();
    uint32_t kept = 0xffffffffu, left = 0u;
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int i = m * kWave + lane;
        if (i < n) {
            if ((bits[i >> 5] >> (i & 31)) & 1u)
                kept = min(kept, key[m]);
            else
                left = max(left, key[m]);
        }
    }
    kept = wave_min_u32(kept);
    left = wave_max_u32(left);
    if (lane == 0)
        boundary_store(P, row, c, kept, left);
}

// Exact selection among compacted candidates sk[0 .. c) (ascending positions), whose
// keys all lie in [t0, kmax]: the bits above the first difference of t0 and kmax
// are common to every candidate, so the threshold search starts below them.
template <int S, typename Emit>
__device__ __forceinline__ void refine_topk(const uint32_t *sk, const int *si, int c, int need, uint32_t t0,
                                            uint32_t kmax, Emit emit)
{
    const int lane = lane_id();
    uint32_t key[S];
#pragma unroll
    for (int m = 0; m < S; m++) {
        const int i = m * kWave + lane;
        key[m] = i < c ? sk[i] : 0u;
    }
    uint32_t tau = t0;
    if (t0 != kmax) {
        const int hb = 31 - __clz(t0 ^ kmax);
        tau = hb == 31 ? 0u : (t0 & ~((2u << hb) - 1u));
        for (int bit = hb; bit >= 0; --bit) {
            const uint32_t cand = tau | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int m = 0; m < S; m++)
                cnt += __popcll(__ballot(m * kWave + lane < c && key[m] >= cand));
            if (cnt >= need)
                tau = cand;
            if (cnt == need)                            // exactly the selection: done
                break;
        }
    }
    int gt = 0;
#pragma unroll
    for (int m = 0; m < S; m++)
        gt += __popcll(__ballot(m * kWave + lane < c && key[m] > tau));
    const int need_eq = need - gt;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int m = 0; m < S; m++) {
        const int i = m * kWave + lane;
        const bool valid = i < c;
        const bool is_gt = valid && key[m] > tau;
        const bool is_eq = valid && key[m] == tau;
        const unsigned long long meq = __ballot(is_eq);
        const int rank = eq_seen + lanes_below(meq);
        eq_seen += __popcll(meq);
        const bool sel = is_gt || (is_eq && rank < need_eq);
        const unsigned long long ms = __ballot(sel);
        const int slot = base + lanes_below(ms);
        if (sel && slot < need)
            emit(slot, si[i]);
        base += __popcll(ms);
    }
}

constexpr int kFilterCap = 512;

// One wavefront, need <= 64: the `need` largest of n keys (layout as wave_topk).
// Every lane holding a key contributes its maximum, and at least need lanes hold
// keys, so the need-th largest key is >= t0 = the smallest lane maximum.  Keys >=
// t0 are compacted in ascending position order into sk/si (kFilterCap entries of
// wavefront-private LDS) and the exact search runs on them alone; more than
// kFilterCap candidates fall back to the full search.
template <int KPL, typename Emit>
__device__ __forceinline__ void wave_topk_filtered(const uint32_t (&key)[KPL], int n, int need, Emit emit,
                                                   uint32_t *sk, int *si)
{
    const int lane = lane_id();
    uint32_t lmax = 0u;
    bool has = false;
#pragma unroll
    for (int m = 0; m < KPL; m++)
        if (m * kWave + lane < n) {
            lmax = max(lmax, key[m]);
            has = true;
        }
    const uint32_t t0 = wave_min_u32(has ? lmax : 0xffffffffu);
    const uint32_t kmax = wave_max_u32(lmax);
    int c = 0;
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int i = m * kWave + lane;
        const bool cnd = i < n && key[m] >= t0;
        const unsigned long long mk = __ballot(cnd);
        const int pos = c + lanes_below(mk);
        if (cnd && pos < kFilterCap) {
            sk[pos] = key[m];
            si[pos] = i;
        }
        c += __popcll(mk);
    }
    if (c > kFilterCap) {
        wave_topk<KPL>(key, n, need, emit);
        return;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (c <= 64)
        refine_topk<1>(sk, si, c, need, t0, kmax, emit);
    else if (c <= 128)
        refine_topk<2>(sk, si, c, need, t0, kmax, emit);
    else if (c <= 256)
        refine_topk<4>(sk, si, c, need, t0, kmax, emit);
    else
        refine_topk<8>(sk, si, c, need, t0, kmax, emit);
}

// The `need` largest of n keys in one wavefront (filtered search for need <= 64).
template <int KPL, typename Emit>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[KPL], int n, int need, Emit emit, uint32_t *sk,
                                            int *si)
{
    if (need <= kWave)
        wave_topk_filtered<KPL>(key, n, need, emit, sk, si);
    else
        wave_topk<KPL>(key, n, need, emit);
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
    if (P.g == 1) {
        const long long row = P.block_table ? (long long)kv_map(P, r.b).row(j) : r.k_off + j;
        return base + (row * P.h_kv + c) * D;
    }
    return base + (((long long)c * P.batch + r.b) * P.nb_max + j) * D;
}

// ---------------------------------------------------------------- score_rows (split)

// Selector slice of this lane: Qs[sub*VPL .. +VPL] summed over the row's queries and
// group c's heads, pair p = (query q_first + p / G, head p % G) added in ascending p.
// The pairs' slices are loaded kSelBatch at a time as raw words: selector_issue
// loads the first batch (called before the key loads, so its latency overlaps
// theirs), selector_finish sums it and loads and sums the rest.
constexpr int kSelBatch = 8;

template <typename T, int VPL>
struct SelBuf {
    static constexpr int W = VPL * (int)sizeof(T) / 4;   // 32-bit words per slice
    uint32_t w[kSelBatch][W];
};

template <typename T, int D, int VPL>
__device__ __forceinline__ void selector_issue(const KP &P, const T *q, const RowGeo &r, int c, int sub,
                                               SelBuf<T, VPL> &buf, int p0 = 0)
{
    constexpr int W = SelBuf<T, VPL>::W;
    const int np = (int)(r.q_last - r.q_first) * P.G;
#pragma unroll
    for (int b = 0; b < kSelBatch; b++) {
        const int p = p0 + b;
        if (p < np) {
            const long long i = r.q_first + p / P.G;
            const T *qi = q + (i * P.h_q + (long long)c * P.G + p % P.G) * D + sub * VPL;
            if constexpr (W == 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(qi);
                buf.w[b][0] = v.x;
                buf.w[b][1] = v.y;
            } else {
                const uint4 v = *reinterpret_cast<const uint4 *>(qi);
                buf.w[b][0] = v.x;
                buf.w[b][1] = v.y;
                buf.w[b][2] = v.z;
                buf.w[b][3] = v.w;
            }
        } else {
#pragma unroll
            for (int x = 0; x < W; x++)
                buf.w[b][x] = 0u;
        }
    }
}

template <typename T, int D, int VPL>
__device__ __forceinline__ void selector_finish(const KP &P, const T *q, const RowGeo &r, int c, int sub,
                                                SelBuf<T, VPL> &buf, float (&qs)[VPL])
{
    constexpr int W = SelBuf<T, VPL>::W;
    static_assert(W == 2 || W == 4, "selector slices of 8 or 16 bytes");
#pragma unroll
    for (int e = 0; e < VPL; e++)
        qs[e] = 0.f;
    const int np = (int)(r.q_last - r.q_first) * P.G;
    for (int p0 = 0; p0 < np; p0 += kSelBatch) {
        if (p0 > 0)
            selector_issue<T, D, VPL>(P, q, r, c, sub, buf, p0);
#pragma unroll
        for (int b = 0; b < kSelBatch; b++) {
            if (p0 + b < np) {
#pragma unroll
                for (int x = 0; x < W; x++) {
                    if constexpr (sizeof(T) == 2) {
                        qs[2 * x] += __uint_as_float(buf.w[b][x] << 16);
                        qs[2 * x + 1] += __uint_as_float(buf.w[b][x] & 0xffff0000u);
                    } else {
                        qs[x] += __uint_as_float(buf.w[b][x]);
                    }
                }
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
// writes order keys to ws[(c*rows+row)*stride + j].  PACKED: workgroup x takes the x-th
// chunk of the rows' actual chunks in row order (a row's chunks cover its candidates;
// rows that keep every candidate have none), so rows far shorter than the longest
// launch no empty workgroups (n_chunk unused).  A variant of its own: the mapping's
// registers would lower the rows x chunks kernel's occupancy (62 -> 77 VGPRs at U = 4).  The loads of round r+1 are
// issued before round r is reduced; the selector slice is built while the first
// round is in flight.  U = 8 key rows per lane group and round; 4 through a block
// table (each key row waits for its page entry, and shorter rounds keep more of
// those two-step loads in the pipeline: 237 against 253 us for the paged drafts).
template <typename T, typename KT, int D, int CH, int U, bool PACKED = false>
__global__ __launch_bounds__(256) void score_rows_kernel(KP P, const T *__restrict__ q,
                                                         const KT *__restrict__ kbase,
                                                         uint32_t *__restrict__ ws, long long stride, int n_chunk)
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 4 * GPW;
    constexpr int RW = U * NG;
    long long row;
    int chunk;
    if constexpr (PACKED) {
        // every wavefront finds the same (row, chunk): the rows' chunk counts, 64 rows
        // at a time, prefix-summed across the lanes
        const int lane = lane_id(), x = (int)blockIdx.x;
        int base = 0;
        row = -1;
        chunk = 0;
        for (int r0 = 0; r0 < P.rows; r0 += kWave) {
            const int rl = r0 + lane;
            int nch = 0;
            if (rl < P.rows) {
                const RowGeo g = row_geo(P, rl);
                nch = g.need == g.n_cand ? 0 : (g.n_cand + CH - 1) / CH;
            }
            int incl = nch;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int t = __shfl_up(incl, o, kWave);
                if (lane >= o)
                    incl += t;
            }
            const int tot = __shfl(incl, kWave - 1, kWave);
            if (x < base + tot) {
                const int l = __ffsll((long long)__ballot(base + incl > x)) - 1;
                row = __builtin_amdgcn_readfirstlane(r0 + l);
                chunk = __builtin_amdgcn_readfirstlane(x - base - (__shfl(incl, l, kWave) - __shfl(nch, l, kWave)));
                break;
            }
            base += tot;
        }
        if (row < 0)
            return;
    } else {
        row = blockIdx.x / n_chunk;
        chunk = (int)(blockIdx.x % n_chunk);
    }
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
    uint32_t *dst = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
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
    SelBuf<T, VPL> sb;
    selector_issue<T, D, VPL>(P, q, r, c, sub, sb);
    load(ra, 0);
    selector_finish<T, D, VPL>(P, q, r, c, sub, sb, qv);
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

// ---------------------------------------------------------------- per-head group scores

// The SOFTMAX and MAX group scores need every head's own score of a block.
// score_heads: grid (rows * n_chunk, h_kv), CH candidates per workgroup.  The
// group's per-head selector queries (head h summed over the row's queries) sit
// in LDS; a key row is read once and dotted with every head, each dot reduced
// over the row's lanes.  MAX writes the order key of the best head's score
// (scaled by 1/sqrt(d)); SOFTMAX writes every head's logit (scaled by 1/tau) to
// ws_l[row][head][j].
constexpr int kMaxG = 64;

template <typename T, typename KT, int D, int CH>
__global__ __launch_bounds__(256) void score_heads_kernel(KP P, const T *__restrict__ q,
                                                          const KT *__restrict__ kbase, uint32_t *__restrict__ ws,
                                                          float *__restrict__ ws_l, long long stride, int n_chunk)
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 4 * GPW;
    constexpr int U = 64 / NG < 1 ? 1 : 64 / NG;          // 64 rows per round
    constexpr int RW = U * NG;
    __shared__ __attribute__((aligned(16))) float sh_q[kMaxG * D];
    const long long row = blockIdx.x / n_chunk;
    const int chunk = (int)(blockIdx.x % n_chunk);
    const int c = blockIdx.y;
    const RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand)                              // every candidate kept: no scores needed
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
            const int j = min(j0 + rd * RW + u * NG + grp, j1 - 1);
            raw[u] = reinterpret_cast<const uint4 *>(key_row<KT, D>(P, kbase, r, c, j))[sub];
        }
    };
    load(ra, 0);
    for (int x = tid; x < P.G * D; x += 256) {
        const long long h = c * P.G + x / D;
        float acc = 0.f;
        for (long long i = r.q_first; i < r.q_last; i++) {
            if constexpr (sizeof(T) == 2)
                acc += bf16_to_f32(q[(i * P.h_q + h) * D + x % D]);
            else
                acc += q[(i * P.h_q + h) * D + x % D];
        }
        sh_q[x] = acc;
    }
    __syncthreads();
    uint32_t *keys = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    float *logits = ws_l + ((long long)c * P.rows + row) * P.G * stride;
    // heads outer, rows inner: one read of a head's query slice per round
    auto reduce = [&](const uint4 (&raw)[U], int rd) {
        float best[U];
#pragma unroll
        for (int u = 0; u < U; u++)
            best[u] = -INFINITY;
        for (int h = 0; h < P.G; h++) {
            float qv[VPL];
#pragma unroll
            for (int e = 0; e < VPL; e++)
                qv[e] = sh_q[h * D + sub * VPL + e];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const float sc = group_sum<L>(slice_dot<VPL>(raw[u], qv)) * P.head_score_scale;
                const int j = j0 + rd * RW + u * NG + grp;
                if (P.select_mode == 2)
                    best[u] = fmaxf(best[u], sc);
                else if (sub == 0 && j < j1)
                    logits[(long long)h * stride + j] = sc;
            }
        }
        if (P.select_mode == 2) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = j0 + rd * RW + u * NG + grp;
                if (sub == 0 && j < j1)
                    keys[j] = order_key(best[u]);
            }
        }
    };
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

// SA_SELECT_ATTN: grid (rows * n_chunk, h_kv).  The row's (query, head) pairs
// (R = its queries x G <= 64) sit in LDS with their log-sum-exps from the verify
// pass; every token of a candidate block is dotted with every pair and
// exp(scale dot - lse) is summed, in a fixed order (the block's tokens, then the
// pairs), into the block's score: the attention mass the verify pass put on it.
template <typename T, int D, int CH>
__global__ __launch_bounds__(256) void score_attn_kernel(KP P, const T *__restrict__ q, const T *__restrict__ k,
                                                         uint32_t *__restrict__ ws, long long stride, int n_chunk)
{
    using RD = RowDot<T, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 4 * GPW;
    constexpr int U = 64 / NG < 1 ? 1 : 64 / NG;          // 64 candidates per round
    constexpr int RW = U * NG;
    __shared__ __attribute__((aligned(16))) float sh_q[kMaxG * D];
    __shared__ float sh_lse[kMaxG];
    const long long row = blockIdx.x / n_chunk;
    const int chunk = (int)(blockIdx.x % n_chunk);
    const int c = blockIdx.y;
    const RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand)
        return;
    const int j0 = r.j_lo + chunk * CH;
    const int j1 = min(j0 + CH, r.j_hi);
    if (j0 >= j1)
        return;
    const int tid = threadIdx.x, lane = lane_id(), sub = lane % L, grp = (tid / kWave) * GPW + lane / L;
    const int R = (int)(r.q_last - r.q_first) * P.G;
    for (int x = tid; x < R * D; x += 256) {
        const int pr = x / D;
        const long long i = r.q_first + pr / P.G;
        const long long h = (long long)c * P.G + pr % P.G;
        if constexpr (sizeof(T) == 2)
            sh_q[x] = bf16_to_f32(q[(i * P.h_q + h) * D + x % D]);
        else
            sh_q[x] = q[(i * P.h_q + h) * D + x % D];
    }
    constexpr float kLog2e = 1.4426950408889634f;
    for (int x = tid; x < R; x += 256) {
        const long long i = r.q_first + x / P.G;
        const long long h = (long long)c * P.G + x % P.G;
        sh_lse[x] = P.attn_lse[h * P.total_q + i] * kLog2e;
    }
    __syncthreads();
    const KvMap kmap = kv_map(P, r.b);
    const T *kb = k + (P.block_table ? 0 : r.k_off * P.h_kv) * D + (long long)c * D;
    uint32_t *keys = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    const int rounds = (j1 - j0 + RW - 1) / RW;
    for (int rd = 0; rd < rounds; rd++) {
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; u++)
            acc[u] = 0.f;
        for (int s = 0; s < P.g; s++) {
            uint4 raw[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int jr = j0 + rd * RW + u * NG + grp;
                const int j = min(jr, j1 - 1);
                const int t = j * P.g + s;
                ok[u] = jr < j1 && t < r.n_k;
                const long long tr = kmap.row(min(t, r.n_k - 1));
                raw[u] = reinterpret_cast<const uint4 *>(kb + tr * P.h_kv * D)[sub];
            }
            for (int pr = 0; pr < R; pr++) {
                float qv[VPL];
#pragma unroll
                for (int e = 0; e < VPL; e++)
                    qv[e] = sh_q[pr * D + sub * VPL + e];
                const float lb = sh_lse[pr];
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const float dot = group_sum<L>(slice_dot<VPL>(raw[u], qv));
                    acc[u] += ok[u] ? exp2f(dot * (P.scale * kLog2e) - lb) : 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + rd * RW + u * NG + grp;
            if (sub == 0 && j < j1)
                keys[j] = order_key(acc[u]);
        }
    }
}

// SA_SELECT_ATTN for token candidates (g = 1) of bf16 keys (d = 128) and rows of at
// most 16 (query, head) pairs -- an S3R refresh after a draft round.  Same grid and
// output as score_attn_kernel; the dot products run on the bf16 matrix cores instead:
// S^T = K Q^T per 16-token chunk (16 tokens x 32 of d per product, the keys loaded
// straight from HBM in operand layout, the row's pairs resident as B operands; bf16
// products are exact and accumulate in fp32, as in the vector kernel's fp32 FMAs).
// Lane (rr, g4) ends with tokens 4 g4 .. 4 g4 + 3 of a chunk against pair rr; each
// takes exp2(s scale log2e - lse) and the 16 pairs of a token are summed by fixed
// 16-lane DPP exchanges.  Wavefront w takes chunks w, w + 4, ... of the workgroup's span,
// U chunks per round, one round's loads in flight while the previous is reduced.
template <int CH>
__global__ __launch_bounds__(256) void score_attn_mfma_kernel(KP P, const uint16_t *__restrict__ q,
                                                              const uint16_t *__restrict__ k,
                                                              uint32_t *__restrict__ ws, long long stride,
                                                              int n_chunk)
{
    constexpr int D = 128, KS = D / 32, U = 2, NWV = 4;
    const long long row = blockIdx.x / n_chunk;
    const int chunk = (int)(blockIdx.x % n_chunk);
    const int c = blockIdx.y;
    const RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand)
        return;
    const int j0 = r.j_lo + chunk * CH;
    const int j1 = min(j0 + CH, r.j_hi);
    if (j0 >= j1)
        return;
    const int lane = lane_id(), w = threadIdx.x / kWave, rr = lane & 15, g4 = lane >> 4;
    const int R = (int)(r.q_last - r.q_first) * P.G;        // <= 16 (checked by the host)
    constexpr float kLog2e = 1.4426950408889634f;
    bf16x8 qop[KS];
    float lb = INFINITY;                                     // pairs past R weigh exp2(-inf) = 0
    if (rr < R) {
        const long long i = r.q_first + rr / P.G;
        const long long h = (long long)c * P.G + rr % P.G;
        const uint16_t *qp = q + (i * P.h_q + h) * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
        lb = P.attn_lse[h * P.total_q + i] * kLog2e;
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const float sc = P.scale * kLog2e;
    const KvMap kmap = kv_map(P, r.b);
    const uint16_t *kb = k + (P.block_table ? 0 : r.k_off * P.h_kv) * D + (long long)c * D + 8 * g4;
    uint32_t *keys = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    const int n16 = (j1 - j0 + 15) / 16;
    const int rounds = (n16 + NWV * U - 1) / (NWV * U);
    u32x4 ra[U][KS], rb[U][KS];
    auto load = [&](u32x4 (&a)[U][KS], int rd) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int ch = (rd * U + u) * NWV + w;
            const int t = min(min(j0 + 16 * ch + rr, j1 - 1), r.n_k - 1);   // g = 1: candidate j is token j
            const uint16_t *kp = kb + (long long)kmap.row(t) * P.h_kv * D;
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                a[u][ks] = ld16(kp + 32 * ks);
        }
    };
    auto reduce = [&](const u32x4 (&a)[U][KS], int rd) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][ks]), qop[ks], sv, 0, 0,
                                                             0);
            float m[4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                m[e] = exp2f(sv[e] * sc - lb);
#pragma unroll
            for (int e = 0; e < 4; e++)
                m[e] = group_sum<16>(m[e]);                   // the 16 pairs of token 4 g4 + e
            const int jb = j0 + 16 * ((rd * U + u) * NWV + w) + 4 * g4;
            if (rr == 0)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if (jb + e < j1)
                        keys[jb + e] = order_key(m[e]);
        }
    };
    load(ra, 0);
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

// Sum over a 256-thread workgroup (or max), in a fixed order: the result does not
// depend on timing.  Every thread gets the result.
template <bool MAX>
__device__ __forceinline__ float block_reduce_256(float v, float *sh)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float u = __shfl_xor(v, o, kWave);
        v = MAX ? fmaxf(v, u) : v + u;
    }
    __syncthreads();                                     // sh is free
    if (lane_id() == 0)
        sh[threadIdx.x / kWave] = v;
    __syncthreads();
    return MAX ? fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3])) : (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// SOFTMAX: grid (rows, h_kv).  Per head h, m_h = max and Z_h = sum of exp(l - m_h)
// over the row's candidates; then S_j = sum_h exp(l_hj - m_h) / Z_h, written as
// order keys for the top-k.
__global__ __launch_bounds__(256) void softmax_rows_kernel(KP P, const float *__restrict__ ws_l,
                                                           uint32_t *__restrict__ ws, long long stride)
{
    __shared__ float sh_red[4];
    __shared__ float sh_m[kMaxG], sh_zi[kMaxG];
    const long long row = blockIdx.x;
    const int c = blockIdx.y, tid = threadIdx.x;
    const RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand)
        return;
    const float *lrow = ws_l + ((long long)c * P.rows + row) * P.G * stride;
    for (int h = 0; h < P.G; h++) {
        const float *l = lrow + (long long)h * stride;
        float m = -INFINITY;
        for (int j = r.j_lo + tid; j < r.j_hi; j += 256)
            m = fmaxf(m, l[j]);
        m = block_reduce_256<true>(m, sh_red);
        float z = 0.f;
        for (int j = r.j_lo + tid; j < r.j_hi; j += 256)
            z += expf(l[j] - m);
        z = block_reduce_256<false>(z, sh_red);
        if (tid == 0) {
            sh_m[h] = m;
            sh_zi[h] = 1.0f / z;
        }
    }
    __syncthreads();
    uint32_t *keys = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    for (int j = r.j_lo + tid; j < r.j_hi; j += 256) {
        float sc = 0.f;
        for (int h = 0; h < P.G; h++)
            sc += expf(lrow[(long long)h * stride + j] - sh_m[h]) * sh_zi[h];
        keys[j] = order_key(sc);
    }
}

// ---------------------------------------------------------------- select_part + select_merge

// Rows with at most 64*KPL candidates and few rows (decode).  select_part: the
// candidates of a row are scored by ceil(n_cand / kPartCand) workgroups of 256
// threads (four share a compute unit, so the loads of the whole table are in
// flight at once); each keeps its part's `need` best (ascending position) as
// (order key, position) pairs in the workspace.  select_merge: one wavefront per
// row selects the row's `need` best among the parts' survivors, which contain it.
constexpr int kPartCand = 128;
constexpr int kRowMaxCand = 1024;   // candidates of a row that the part and row plans hold

// A part keeps its need + 1 best: the union of the parts' survivors then holds the row's
// need best and its (need+1)-th (every key above that one is among the need best).
__host__ __device__ inline int part_cap(int topk) { return topk < kPartCand ? topk + 1 : kPartCand; }

template <typename T, typename KT, int D>
__global__ __launch_bounds__(256) void select_part_kernel(KP P, const T *__restrict__ q,
                                                          const KT *__restrict__ kbase, uint32_t *__restrict__ ws_k,
                                                          int32_t *__restrict__ ws_i, int n_part)
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = 4 * GPW;
    constexpr int U = (kPartCand + NG - 1) / NG;
    __shared__ uint32_t sh_key[kPartCand];
    __shared__ uint32_t sh_k[kFilterCap];
    __shared__ int sh_i[kFilterCap];
    const long long row = blockIdx.x / n_part;
    const int part = (int)(blockIdx.x % n_part);
    const int c = blockIdx.y;
    const int tid = threadIdx.x, lane = lane_id(), sub = lane % L, grp = (tid / kWave) * GPW + lane / L;
    RowGeo r = row_geo(P, row);
    if (r.need == r.n_cand || r.need == 0)                // the merge writes these rows alone
        return;
    const int i0 = part * kPartCand, i1 = min(i0 + kPartCand, r.n_cand);
    if (i0 >= i1)
        return;
    SelBuf<T, VPL> sb;
    selector_issue<T, D, VPL>(P, q, r, c, sub, sb);
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int i = min(i0 + u * NG + grp, i1 - 1);
        raw[u] = reinterpret_cast<const uint4 *>(key_row<KT, D>(P, kbase, r, c, r.j_lo + i))[sub];
    }
    float qv[VPL];
    selector_finish<T, D, VPL>(P, q, r, c, sub, sb, qv);
#pragma unroll
    for (int u = 0; u < U; u++) {
        const float sc = group_sum<L>(slice_dot<VPL>(raw[u], qv));
        const int i = u * NG + grp;
        if (sub == 0 && i0 + i < i1)
            sh_key[i] = order_key(sc);
    }
    __syncthreads();
    if (tid >= kWave)
        return;
    const int n = i1 - i0, cap = part_cap(P.topk);
    const long long slot0 = (((long long)c * P.rows + row) * n_part + part) * cap;
    uint32_t kr[kPartCand / kWave];
#pragma unroll
    for (int m = 0; m < kPartCand / kWave; m++) {
        const int i = m * kWave + lane;
        kr[m] = i < n ? sh_key[i] : 0u;
    }
    const int keep = min(r.need + 1, n);
    if (keep == n) {                                     // the whole part survives
        for (int i = lane; i < n; i += kWave) {
            ws_k[slot0 + i] = sh_key[i];
            ws_i[slot0 + i] = i0 + i;
        }
        return;
    }
    auto emit = [&](int slot, int i) {
        ws_k[slot0 + slot] = sh_key[i];
        ws_i[slot0 + slot] = i0 + i;
    };
    wave_select<kPartCand / kWave>(kr, n, keep, emit, sh_k, sh_i);
}

// 4 wavefronts per workgroup, one row each.  grid: (ceil(rows / 4), h_kv).
template <int KPL>
__global__ __launch_bounds__(256) void select_merge_kernel(KP P, const uint32_t *__restrict__ ws_k,
                                                           const int32_t *__restrict__ ws_i, int n_part,
                                                           int32_t *__restrict__ idx, int32_t *__restrict__ n_idx)
{
    __shared__ uint32_t sh_k[4][kFilterCap];
    __shared__ int sh_i[4][kFilterCap];
    __shared__ int sh_pos[4][64 * KPL];
    __shared__ uint32_t sh_bits[4][2 * KPL];
    const long long row = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    const int c = blockIdx.y, lane = lane_id(), wv = threadIdx.x / kWave;
    if (row >= P.rows)
        return;
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (lane == 0) {
        n_idx[(long long)c * P.rows + row] = r.need;
        if (P.boundary && (r.need == r.n_cand || r.need == 0))
            boundary_none(P, row, c);
    }
    if (r.need == r.n_cand) {
        write_all(P, out, r, lane, kWave);
        return;
    }
    if (r.need == 0) {
        for (int s2 = lane; s2 < P.topk; s2 += kWave)
            out[s2] = -1;
        return;
    }
    // survivors: full parts keep m_full = min(need + 1, kPartCand), the last part m_last
    const int cap = part_cap(P.topk);
    const int n_part_row = (r.n_cand + kPartCand - 1) / kPartCand;
    const int m_full = min(r.need + 1, kPartCand);
    const int m_last = min(r.need + 1, r.n_cand - (n_part_row - 1) * kPartCand);
    const int m_tot = (n_part_row - 1) * m_full + m_last;
    const long long base = ((long long)c * P.rows + row) * n_part * cap;
    uint32_t kr[KPL];
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int j = m * kWave + lane;
        const int pt = j / m_full, sl = j - pt * m_full;
        const long long o = base + (long long)pt * cap + sl;
        kr[m] = j < m_tot ? ws_k[o] : 0u;
        if (j < m_tot)
            sh_pos[wv][j] = ws_i[o];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the survivors are in ascending position order, so selecting among them by their
    // rank keeps the lower block index on equal scores
    const bool audit = P.boundary != nullptr;
    if (audit) {
        if (lane < 2 * KPL)
            sh_bits[wv][lane] = 0u;
        wave_lds_sync();
    }
    auto emit = [&](int slot, int j) {
        out[slot] = r.j_lo + sh_pos[wv][j];
        if (audit)
            mark_selected(sh_bits[wv], j);
    };
    wave_select<KPL>(kr, m_tot, r.need, emit, sh_k[wv], sh_i[wv]);
    for (int s2 = r.need + lane; s2 < P.topk; s2 += kWave)
        out[s2] = -1;
    if (audit) {                                         // the (need+1)-th is a survivor
        wave_lds_sync();
        wave_boundary<KPL>(P, row, c, kr, m_tot, sh_bits[wv]);
    }
}

// The need-th largest of n keys (n >= need >= 1), found by the 16 wavefronts of a
// 1024-thread workgroup that each hold all n keys in registers (key i at lane i % 64,
// slot i / 64).  The bits above `shift + 4` are fixed by tau (every key >= tau, and
// at least need of them); the rest are found 4 bits per round: wavefront w counts the
// keys >= tau | w << shift, the counts meet in LDS (two buffers: one barrier per
// round) and every wavefront takes the largest digit whose count still reaches
// need.  A count of exactly need ends the search early: the keys at or above the
// returned value are then exactly the need largest.
template <int KPL, int NW = 16>
__device__ __forceinline__ uint32_t block_threshold16(const uint32_t (&kr)[KPL], int n, int need, uint32_t tau,
                                                      int shift, int (*sh_cnt)[16])
{
    static_assert(16 % NW == 0, "wavefronts must divide the 16 digits of a round");
    const int lane = lane_id(), w = threadIdx.x / kWave;
    for (int rd = 0; shift >= 0; rd++, shift -= 4) {
        // with NW < 16 wavefronts, wavefront w counts digits w, w + NW, ...
#pragma unroll
        for (int j = 0; j < 16 / NW; j++) {
            const uint32_t cand = tau | ((uint32_t)(w + j * NW) << shift);
            int cnt = 0;
#pragma unroll
            for (int m = 0; m < KPL; m++)
                cnt += __popcll(__ballot(m * kWave + lane < n && kr[m] >= cand));
            if (lane == 0)
                sh_cnt[rd & 1][w + j * NW] = cnt;
        }
        __syncthreads();
        const int cl = sh_cnt[rd & 1][lane & 15];
        // digit 0 keeps tau itself, which always has >= need keys at or above it
        const unsigned long long ok = __ballot(lane < 16 && cl >= need);
        const int d = 63 - __clzll(ok);
        tau |= (uint32_t)d << shift;
        if (__builtin_amdgcn_readlane(cl, d) == need)
            break;
    }
    return tau;
}

// Selection among a row's n <= 64 * KPL keys in LDS by the 16 wavefronts of a
// workgroup: the threshold by block_threshold16, then wavefront 0 emits the
// selection in ascending index (keys above it, then the lowest-index keys equal to it).
template <int KPL, int NW = 16>
__device__ __forceinline__ void row_select(const KP &P, const uint32_t *sh_key, int (*sh_cnt)[16], const RowGeo &r,
                                           int32_t *out, int32_t *n_idx_row, uint32_t *sh_bits, long long row, int c,
                                           int *lds_sel)
{
    const int lane = lane_id(), n = r.n_cand, need = r.need;
    uint32_t kr[KPL];
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int i = m * kWave + lane;
        kr[m] = i < n ? sh_key[i] : 0u;
    }
    const uint32_t tau = block_threshold16<KPL, NW>(kr, n, need, 0u, 28, sh_cnt);
    if (threadIdx.x >= kWave)
        return;
    if (lane == 0)
        *n_idx_row = need;
    const bool audit = P.boundary != nullptr;
    if (audit) {
        for (int x = lane; x < 2 * KPL; x += kWave)
            sh_bits[x] = 0u;
        wave_lds_sync();
    }
    emit_above<KPL>(kr, n, need, tau, [&](int slot, int i) {
        out[slot] = r.j_lo + i;
        if (lds_sel)
            lds_sel[slot] = r.j_lo + i;
        if (audit)
            mark_selected(sh_bits, i);
    });
    for (int s2 = need + lane; s2 < P.topk; s2 += kWave)
        out[s2] = -1;
    if (audit) {
        wave_lds_sync();
        wave_boundary<KPL>(P, row, c, kr, n, sh_bits);
    }
}

// One workgroup of 16 wavefronts per (row, KV head), for batches whose rows x KV
// heads give every CU a workgroup: the row's candidates are scored into LDS in
// passes of kRowPass (U rounds of 16 x GPW key rows, all loads of a pass issued
// before any is reduced), then wavefront 0 selects the row's need best.  Same
// per-candidate arithmetic as select_part; no workspace and one launch instead of
// part + merge.  grid: rows x h_kv, the KV head fastest.
constexpr int kRowPass = 512;

// The row plan's work for (row, KV head c), called by all NW * 64 threads of the
// workgroup: the step's append for the row's sequence (app.n_blk > 0), the row's
// candidates scored into sh_key, the selection written to idx / n_idx (and to
// lds_sel, in ascending order, when given), the audit when asked.  before_search()
// runs on every thread once the keys are scored (after the append and a barrier),
// before the threshold search, when the row ranks its candidates.  Returns the
// row's selection count.  The threads return from it at different points: a
// caller that goes on must meet at a barrier first.
struct NoHook {
    __device__ void operator()() const {}
};

template <typename T, typename KT, int D, int NW = 16, typename Hook = NoHook>
__device__ __forceinline__ int row_plan_select(const KP &P, const T *__restrict__ q, const KT *__restrict__ kbase,
                                               int32_t *__restrict__ idx, int32_t *__restrict__ n_idx,
                                               const SelAppend &app, long long row, int c, uint32_t *sh_key,
                                               uint32_t *sh_bits, int (*sh_cnt)[16], int *lds_sel,
                                               Hook before_search = Hook())
{
    using RD = RowDot<KT, D>;
    constexpr int L = RD::L, VPL = RD::VPL;
    constexpr int GPW = kWave / L, NG = NW * GPW;
    constexpr int U = kRowPass / NG;
    const int tid = threadIdx.x, lane = lane_id(), sub = lane % L, grp = (tid / kWave) * GPW + lane / L;
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    // the step's append for this row's sequence and KV head (one query per sequence):
    // its new token's rows and the blocks whose pooling window holds it, none of which
    // is a candidate of the row (the launcher checks window >= block).  It runs first:
    // run beside the key loads in flight, its registers spill (with 16 wavefronts) or
    // it costs more than it hides (8 wavefronts of the decode step: 82.6 against 75.8 us).
    auto append = [&]() {
        if (app.n_blk == 0)
            return;
        const int b = seq_of_query(P, row);
        const T *kn = (const T *)app.k_new, *vn = (const T *)app.v_new;
        T *kw = (T *)app.k, *vw = (T *)app.v;
        for (int jj = 0; jj < app.n_blk; jj++) {
            const long long item = ((long long)b * P.h_kv + c) * app.n_blk + jj;
            if (P.pool == 1)
                append_pool_item<T, D, 1>(P, kn, vn, kw, vw, app.k_cmp, app.n_blk, item);
            else
                append_pool_item<T, D, 0>(P, kn, vn, kw, vw, app.k_cmp, app.n_blk, item);
        }
    };
    append();
    if (r.need == r.n_cand || r.need == 0) {
        if (tid == 0) {
            n_idx[(long long)c * P.rows + row] = r.need;
            if (P.boundary)
                boundary_none(P, row, c);
        }
        if (r.need == 0)
            for (int s2 = tid; s2 < P.topk; s2 += blockDim.x)
                out[s2] = -1;
        else
            write_all(P, out, r, tid, blockDim.x);
        if (lds_sel)
            for (int s2 = tid; s2 < r.need; s2 += blockDim.x)
                lds_sel[s2] = r.j_lo + s2;
        return r.need;
    }
    float qv[VPL];
    SelBuf<T, VPL> sb;
    selector_issue<T, D, VPL>(P, q, r, c, sub, sb);
    for (int p0 = 0; p0 < r.n_cand; p0 += kRowPass) {
        const int i1 = min(p0 + kRowPass, r.n_cand);
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = min(p0 + u * NG + grp, i1 - 1);
            raw[u] = reinterpret_cast<const uint4 *>(key_row<KT, D>(P, kbase, r, c, r.j_lo + i))[sub];
        }
        if (p0 == 0)
            selector_finish<T, D, VPL>(P, q, r, c, sub, sb, qv);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float sc = group_sum<L>(slice_dot<VPL>(raw[u], qv));
            const int i = p0 + u * NG + grp;
            if (sub == 0 && i < i1)
                sh_key[i] = order_key(sc);
        }
    }
    __syncthreads();
    before_search();
    if (r.n_cand <= 8 * kWave)
        row_select<8, NW>(P, sh_key, sh_cnt, r, out, n_idx + (long long)c * P.rows + row, sh_bits, row, c, lds_sel);
    else
        row_select<kRowMaxCand / kWave, NW>(P, sh_key, sh_cnt, r, out, n_idx + (long long)c * P.rows + row,
                                            sh_bits, row, c, lds_sel);
    return r.need;
}

template <typename T, typename KT, int D>
__global__ __launch_bounds__(1024) void select_row_kernel(KP P, const T *__restrict__ q,
                                                          const KT *__restrict__ kbase, int32_t *__restrict__ idx,
                                                          int32_t *__restrict__ n_idx, SelAppend app)
{
    __shared__ uint32_t sh_key[kRowMaxCand];
    __shared__ uint32_t sh_bits[kRowMaxCand / 32];
    __shared__ int sh_cnt[2][16];
    // consecutive workgroups take the KV heads of one row (each XCD serves one head):
    // 19.9 against 21.5 us per decode selection with rows in consecutive workgroups
    row_plan_select<T, KT, D>(P, q, kbase, idx, n_idx, app, blockIdx.x / P.h_kv, blockIdx.x % P.h_kv, sh_key, sh_bits,
                              sh_cnt, nullptr);
}

// ---------------------------------------------------------------- decode step (one launch)

// A decode step in one launch for (row = sequence, KV head c): the row plan's append
// and selection (row_plan_select on 8 wavefronts: the same arithmetic and results as
// the 16-wavefront row kernel, with all of the row's key loads in flight at once),
// then attention over the row's set by the 8 wavefronts with the selection read from
// LDS.  Each wavefront walks 32-token chunks with the gather kernel's load/compute
// steps, the next chunk's loads in flight while one is computed (16 chunks per
// compute unit); the wavefronts' (max, sum, output) partials are merged through LDS
// in wavefront order.  The host checks: bf16, one query per sequence, pooled keys,
// G <= kStepRows, the set fits the LDS token list.
constexpr int kStepRows = 8;
constexpr int kStepWaves = 8;

template <int D>
__global__ __launch_bounds__(kStepWaves * 64) void decode_step_kernel(KP P, const uint16_t *__restrict__ q,
                                                           const float *__restrict__ k_cmp,
                                                           const uint16_t *k,    // written too (the append)
                                                           const uint16_t *v,
                                                           int32_t *__restrict__ idx, int32_t *__restrict__ n_idx,
                                                           uint16_t *__restrict__ out, float *__restrict__ lse,
                                                           SelAppend app)
{
    constexpr int KS = D / 32;
    __shared__ uint32_t sh_key[kRowMaxCand];
    __shared__ uint32_t sh_bits[kRowMaxCand / 32];
    __shared__ int sh_cnt[2][16];
    __shared__ int sh_sel[kRowMaxCand];
    __shared__ float sh_m[kStepWaves][kStepRows], sh_l[kStepWaves][kStepRows];
    __shared__ int sh_buf[kTokCap > kStepWaves * kStepRows * D ? kTokCap : kStepWaves * kStepRows * D];
    // (the token list, then the wavefronts' outputs)
    __shared__ int sh_pre[32 * kStepWaves];                  // rows of the fixed positions loaded early
    __shared__ float sh_app[2048];                           // the append's partial sums (TG x D)
    // consecutive workgroups take the KV heads of one row: the XCDs (which receive
    // workgroups in turn) each serve one head
    const long long row = blockIdx.x / P.h_kv;
    const int c = blockIdx.x % P.h_kv, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int rr = lane & 15, g4 = lane >> 4;
    const int b = seq_of_query(P, row);
    const Seq s = seq_info(P, b);
    const int p = s.q0 + (int)(row - s.q_off);
    const KvMap kmap = kv_map(P, b);
    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (kv_base(P, s) * P.h_kv + c) * D;
    const uint16_t *vb = v + (kv_base(P, s) * P.h_kv + c) * D;
    // The attended list runs init | window | selected blocks (the softmax does not
    // depend on the order).  Its first n_fix positions (init and window) are known
    // before the selection: their first chunks are loaded while the selection's
    // threshold search runs, when HBM would otherwise idle.
    const ASet a0 = aset_make(P, s.n_k, p, p, nullptr, 0);
    const int n_fix = a0.n1 + a0.n3;
    const int n_pre = min(n_fix, 32 * kStepWaves);
    for (int x = tid; x < n_pre; x += blockDim.x)
        sh_pre[x] = kmap.row(aset_token(a0, nullptr, x));   // no selection: init, then window
    // The step's append (the new token's cache rows, the re-pooled block that holds it)
    // feeds no candidate of this selection (the block lies in the window), only the
    // attention, which reads the new token: its loads go out with the prefetch, before
    // the threshold search, and it is finished after the selection.  Run first, it held
    // back every score load by its memory latency (about 6 us of a 72 us step).
    const bool defer = app.n_blk > 0 && append_split_fits<D>(P);
    SelAppend app_sel = app;
    if (defer)
        app_sel.n_blk = 0;
    AppendSplit<D> aps;
    uint4 aps_knew, aps_vnew;
    long long aps_crow = -1;
    bool aps_issued = false;
    ChunkRegs<D> ra, rb;
    bool loaded = false;                                      // ra holds this wavefront's first chunk
    auto prefetch = [&]() {
        if (defer) {
            append_split_issue<D, 4>(P, s, kmap, (const uint16_t *)app.k_new, (const uint16_t *)app.v_new, k,
                                     app.n_blk, c, aps, aps_knew, aps_vnew, aps_crow);
            aps_issued = true;
        }
        // the chunk lies wholly in the fixed part (and, with the append still to come,
        // before its last entry, the new token)
        if (32 * w + 32 <= n_pre && (!defer || 32 * w + 32 < n_fix)) {
            load_chunk<D>(ra, sh_pre, 32 * w, n_pre, kb, vb, tstride, rr, g4, n_pre);
            loaded = true;
        }
    };
    const int nsel = row_plan_select<uint16_t, float, D, kStepWaves>(P, q, k_cmp, idx, n_idx, app_sel, row, c,
                                                                     sh_key, sh_bits, sh_cnt, sh_sel, prefetch);
    if (defer) {
        if (!aps_issued)                                      // a row that ranks nothing skips the hook
            append_split_issue<D, 4>(P, s, kmap, (const uint16_t *)app.k_new, (const uint16_t *)app.v_new, k,
                                     app.n_blk, c, aps, aps_knew, aps_vnew, aps_crow);
        if (P.pool == 1)
            append_split_commit<D, 4, 1>(aps, aps_knew, aps_vnew, aps_crow, (uint16_t *)app.k, (uint16_t *)app.v,
                                         sh_app);
        else
            append_split_commit<D, 4, 0>(aps, aps_knew, aps_vnew, aps_crow, (uint16_t *)app.k, (uint16_t *)app.v,
                                         sh_app);
    }
    // the append wrote this sequence's new rows for head c, which the set reaches (its
    // window ends at the query); this workgroup alone reads them back, and the barrier's
    // workgroup-scope fences make its own stores visible to all its wavefronts (one
    // compute unit, one L1).  A device-scope fence here would write back and invalidate
    // the L2 once per workgroup (measured: +30 us per step).
    __syncthreads();
    if (defer) {
        if (P.pool == 1)
            append_split_store<D, 4, 1>(P, aps, app.k_cmp, b, c, sh_app);
        else
            append_split_store<D, 4, 0>(P, aps, app.k_cmp, b, c, sh_app);
    }

    const ASet a = aset_make(P, s.n_k, p, p, sh_sel, nsel);
    const int n = a.total;                                   // <= kTokCap (checked by the host)
    int *sh_tok = sh_buf;
    for (int x = tid; x < n; x += blockDim.x)
        sh_tok[x] = kmap.row(aset_token(a, sh_sel, x < n_fix ? (x < a.n1 ? x : x + a.n2) : x - a.n3));
    const int R = P.G;
    bf16x8 qop[KS];
    if (rr < R) {
        const uint16_t *qp = q + (row * P.h_q + c * P.G + rr) * D + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();

    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int pp = 0; pp < 8; pp++)
        acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (32 * w < n && !loaded)
        load_chunk<D>(ra, sh_tok, 32 * w, n, kb, vb, tstride, rr, g4, n);
    for (int ch = w; 32 * ch < n; ch += 2 * kStepWaves) {
        const int c1 = ch + kStepWaves;
        if (32 * c1 < n)
            load_chunk<D>(rb, sh_tok, 32 * c1, n, kb, vb, tstride, rr, g4, n);
        compute_chunk<D>(ra, ra.live, qop, P.scale_log2, g4, m_run, l_part, acc);
        if (32 * c1 >= n)
            break;
        const int c2 = c1 + kStepWaves;
        if (32 * c2 < n)
            load_chunk<D>(ra, sh_tok, 32 * c2, n, kb, vb, tstride, rr, g4, n);
        compute_chunk<D>(rb, rb.live, qop, P.scale_log2, g4, m_run, l_part, acc);
    }
    float l_row = l_part + __shfl_xor(l_part, 16, kWave);
    l_row += __shfl_xor(l_row, 32, kWave);
    __syncthreads();                                         // every wavefront is done with the token list
    float *sh_o = reinterpret_cast<float *>(sh_buf);         // [waves][rows < R][D]
    if (g4 == 0 && rr < R) {
        sh_m[w][rr] = m_run;
        sh_l[w][rr] = l_row;
    }
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
        const int rw = 4 * g4 + qq;
        if (rw < R && (D == 128 || rr < D / 8)) {
            float *dst = sh_o + (w * kStepRows + rw) * D + 8 * rr;
#pragma unroll
            for (int pp = 0; pp < 8; pp++)
                dst[pp] = acc[pp][qq];
        }
    }
    __syncthreads();
    for (int it = tid; it < R * D; it += blockDim.x) {
        const int r = it / D, e = it % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kStepWaves; ww++)
            M = fmaxf(M, sh_m[ww][r]);
        float Ls = 0.f, O = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < kStepWaves; ww++) {
                const float f = exp2f(sh_m[ww][r] - M);
                Ls += sh_l[ww][r] * f;
                O += sh_o[(ww * kStepRows + r) * D + e] * f;
            }
        }
        const int h = c * P.G + r;
        out[(row * P.h_q + h) * D + e] = f32_to_bf16(O / Ls);
        if (lse && e == 0)
            lse[(long long)h * P.total_q + row] = (M + log2f(Ls)) * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------- score_tile (MFMA fp32)

// 4 consecutive candidate-key elements as fp32 (pooled fp32 keys, or raw bf16 / fp32 keys).
__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 ld4f(const uint16_t *p)
{
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
}

// Prefill rows (one per query).  grid: (column chunks of col_tiles x 64 candidates,
// row tiles of 64, h_kv * batch).  4 wavefronts in 2 x 2, each a 32 x 32 block of
// 2 x 2 MFMA 16x16x4 f32 tiles.  The selector-query operands (the group's heads
// summed in fp32) are built once per workgroup and stay in registers.  Key tiles
// (64 candidate rows) go through a two-buffer LDS ring shared by the four
// wavefronts: while tile t is computed from LDS, tile t+1 is written from
// registers into the other buffer and the loads of tile t+2 are in flight (one
// barrier per tile).  Operand lane l reads key row l%16, head-dim elements
// 16k + 4(l/16) .. +4 (the MFMA k index l/16 of the four steps s = 0..3).  The head
// dimension is contracted in the order (k, s, l/16); fp32 products and sums.
// Column tiles per workgroup: at least 16, more when there are few row tiles (long
// rows, few queries), so each workgroup builds its selector operands for more work
// while the grid still holds >= 2048 workgroups.
static int score_col_tiles(long long stride, long long row_tiles)
{
    const long long n_tiles = (stride + 63) / 64;
    const long long chunks = std::max(1LL, 2048 / std::max(1LL, row_tiles));
    return (int)std::max(16LL, (n_tiles + chunks - 1) / chunks);
}

__device__ __forceinline__ float4 lds4f(const unsigned char *p, float) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 lds4f(const unsigned char *p, uint16_t)
{
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
}

// A thread's share of one staged 64-row key tile (pieces tid + 256 u, 16 bytes each);
// a native vector type, so the copies stay in registers.
typedef uint32_t kv4u __attribute__((ext_vector_type(4)));
template <int N>
struct KeyStage {
    kv4u c[N];
};

// Candidate row j lives at base + map.row(j) * row_stride (raw keys may be paged).
template <int N, int kRowBytes>
__device__ __forceinline__ void key_issue(KeyStage<N> &st, const unsigned char *base, long long row_stride,
                                          const KvMap &map, int jt, int j_end, int tid)
{
#pragma unroll
    for (int u = 0; u < N; u++) {
        const int piece = tid + 256 * u, row = piece / (kRowBytes / 16), col = piece % (kRowBytes / 16);
        const int j = min(jt + row, j_end - 1);          // rows past the end re-read the last one
        st.c[u] = *reinterpret_cast<const kv4u *>(base + (long long)map.row(j) * row_stride + 16 * col);
    }
}

template <int N, int kRowBytes, int kPitch>
__device__ __forceinline__ void key_write(const KeyStage<N> &st, unsigned char *buf, int tid)
{
#pragma unroll
    for (int u = 0; u < N; u++) {
        const int piece = tid + 256 * u, row = piece / (kRowBytes / 16), col = piece % (kRowBytes / 16);
        *reinterpret_cast<kv4u *>(buf + row * kPitch + 16 * col) = st.c[u];
    }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Maxima of 8 values over each 16-lane row, transposed: v[t] (t = 0..7) of all 16
// lanes reduce to lane l holding the maximum of v[l & 7].  Each exchange step halves
// the values a lane holds: the lane keeps the half its lane bit selects and sends
// the other half to a partner whose bit differs (xor 1, xor 2 by quad permutes;
// rotations by 4 and 8 lanes flip bits 2 and 3).
__device__ __forceinline__ uint32_t row16_max8(const uint32_t (&v)[8], int li)
{
    uint32_t a[4], b[2];
    const bool b0 = li & 1, b1 = li & 2, b2 = li & 4;
#pragma unroll
    for (int p = 0; p < 4; p++)
        a[p] = max(b0 ? v[2 * p + 1] : v[2 * p], dpp_u32<0xB1>(b0 ? v[2 * p] : v[2 * p + 1]));
#pragma unroll
    for (int p = 0; p < 2; p++)          // a[p] holds t = 2p + bit0
        b[p] = max(b1 ? a[2 * p + 1] : a[2 * p], dpp_u32<0x4E>(b1 ? a[2 * p] : a[2 * p + 1]));
    uint32_t c = max(b2 ? b[1] : b[0], dpp_u32<0x124>(b2 ? b[0] : b[1]));   // t = 4 bit2 + 2 bit1 + bit0
    return max(c, dpp_u32<0x128>(c));
}

// With gmax: also the largest order key of every group of kGroupCols consecutive
// candidates (group x = candidates first_cand + 32x ..; 0 where a row has none),
// gmax[(c * rows + row) * gstride + x], so a top-k over long rows can skip the groups
// that cannot hold a selected key.  Each wavefront's 32 columns of a tile are one group.
constexpr int kGroupCols = 32;

template <typename T, typename KT, int D>
__global__ __launch_bounds__(256, 2) void score_tile_kernel(KP P, const T *__restrict__ q,
                                                            const KT *__restrict__ kbase,
                                                            uint32_t *__restrict__ ws, long long stride,
                                                            int col_tiles, uint32_t *__restrict__ gmax,
                                                            long long gstride)
{
    constexpr int KG = D / 16;
    constexpr int kRowBytes = D * (int)sizeof(KT);       // one candidate key row
    constexpr int kPitch = kRowBytes + 16;               // LDS row pitch: 16 rows hit 16 bank groups
    constexpr int kChunks = 64 * kRowBytes / 16 / 256;   // 16-byte pieces per thread per tile
    __shared__ __attribute__((aligned(16))) unsigned char sh_k[2][64 * kPitch];
    const int b = blockIdx.z % P.batch, c = blockIdx.z / P.batch;
    const Seq s = seq_info(P, b);
    const int r0 = blockIdx.y * 64;
    if (r0 >= s.n_q)
        return;
    const int r_end = min(r0 + 64, s.n_q);
    int jlo_last, jhi_last;
    row_cands(P, s.n_k, s.q0 + r_end - 1, jlo_last, jhi_last);
    jhi_last = min(jhi_last, (int)stride);
    const int jc_base = jlo_last;                         // = first_cand for a row with candidates
    const int jc0 = jc_base + blockIdx.x * col_tiles * 64;
    if (jc0 >= jhi_last)
        return;
    const int jc1 = min(jc0 + col_tiles * 64, jhi_last);
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int li = lane % 16, lk = lane / 16;
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;

    // selector operands: rows r0 + wr + 16a + li, elements 16k + 4lk .. +4
    float4 qa[2][KG];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        const int rl = r0 + wr + 16 * a + li;
#pragma unroll
        for (int k = 0; k < KG; k++)
            qa[a][k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rl < r_end) {
            const long long i = s.q_off + rl;
            for (int h = 0; h < P.G; h++) {
                const T *qp = q + (i * P.h_q + (long long)c * P.G + h) * D + 4 * lk;
#pragma unroll
                for (int k = 0; k < KG; k++) {
                    float4 x = ld4f(qp + 16 * k);
                    qa[a][k].x += x.x;
                    qa[a][k].y += x.y;
                    qa[a][k].z += x.z;
                    qa[a][k].w += x.w;
                }
            }
        }
    }
    // candidate upper bound of each output row this lane writes (rows are fixed per workgroup);
    // the lower bound n_init / g is the same for every row that has candidates
    int jh_row[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int rl = r0 + wr + 16 * a + 4 * lk + i;
            int jl = 0, jh = 0;
            if (rl < r_end)
                row_cands(P, s.n_k, s.q0 + rl, jl, jh);
            jh_row[a][i] = jh > jl ? min(jh, (int)stride) : 0;
        }
    const int j_first = first_cand(P);
    // staging: thread tid holds pieces tid + 256 u of the tile (row = piece / pieces per row)
    const unsigned char *kbytes = reinterpret_cast<const unsigned char *>(kbase);
    const long long row_stride = P.g == 1 ? (long long)P.h_kv * kRowBytes : kRowBytes;
    const long long base_off = P.g == 1 ? (kv_base(P, s) * P.h_kv + c) * kRowBytes
                                        : (((long long)c * P.batch + b) * P.nb_max) * kRowBytes;
    const unsigned char *kb0 = kbytes + base_off;
    const KvMap kmap = P.g == 1 ? kv_map(P, b) : KvMap{nullptr, 0};
    auto tile = [&](const unsigned char *buf, int jt) {
        floatx4 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int bb = 0; bb < 2; bb++)
                acc[a][bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KG; k++) {
            float bv[2][4];
#pragma unroll
            for (int bb = 0; bb < 2; bb++) {
                const float4 x = lds4f(buf + (wc + 16 * bb + li) * kPitch + (16 * k + 4 * lk) * (int)sizeof(KT), KT{});
                bv[bb][0] = x.x;
                bv[bb][1] = x.y;
                bv[bb][2] = x.z;
                bv[bb][3] = x.w;
            }
            const float av[2][4] = {{qa[0][k].x, qa[0][k].y, qa[0][k].z, qa[0][k].w},
                                    {qa[1][k].x, qa[1][k].y, qa[1][k].z, qa[1][k].w}};
#pragma unroll
            for (int st = 0; st < 4; st++)
#pragma unroll
                for (int a = 0; a < 2; a++)
#pragma unroll
                    for (int bb = 0; bb < 2; bb++)
                        acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a][st], bv[bb][st], acc[a][bb], 0, 0, 0);
        }
        // row = r0 + wr + 16a + 4lk + i, candidate = jt + wc + 16bb + li
        uint32_t mx[8];
#pragma unroll
        for (int a = 0; a < 2; a++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int rl = r0 + wr + 16 * a + 4 * lk + i;
                uint32_t *dst = ws + ((long long)c * P.rows + s.q_off + rl) * stride + key_col0(P);
                mx[4 * a + i] = 0u;
#pragma unroll
                for (int bb = 0; bb < 2; bb++) {
                    const int j = jt + wc + 16 * bb + li;
                    const uint32_t key = order_key(acc[a][bb][i]);
                    const bool ok = j >= j_first && j < jh_row[a][i];
                    if (ok)
                        dst[j] = key;
                    mx[4 * a + i] = max(mx[4 * a + i], ok ? key : 0u);
                }
            }
        }
        if (gmax && jt + wc < jc1) {                         // groups past the chunk hold no candidate
            const uint32_t m = row16_max8(mx, li);           // row t = li & 7: a = t / 4, i = t % 4
            const int t = li & 7, rl = r0 + wr + 16 * (t >> 2) + 4 * lk + (t & 3);
            if (li < 8 && rl < r_end)
                gmax[((long long)c * P.rows + s.q_off + rl) * gstride + (unsigned)(jt + wc - jc_base) / kGroupCols] = m;
        }
    };
    const int n_t = (jc1 - jc0 + 63) / 64;
    KeyStage<kChunks> stage;
    key_issue<kChunks, kRowBytes>(stage, kb0, row_stride, kmap, jc0, jhi_last, tid);
    key_write<kChunks, kRowBytes, kPitch>(stage, sh_k[0], tid);
    key_issue<kChunks, kRowBytes>(stage, kb0, row_stride, kmap, jc0 + 64, jhi_last, tid);   // past the end: reloads
    for (int t = 0; t < n_t; t++) {
        __syncthreads();                                  // buffer t&1 holds tile t
        tile(sh_k[t & 1], jc0 + 64 * t);
        key_write<kChunks, kRowBytes, kPitch>(stage, sh_k[(t + 1) & 1], tid);
        key_issue<kChunks, kRowBytes>(stage, kb0, row_stride, kmap, jc0 + 64 * (t + 2), jhi_last, tid);
    }
}

// ---------------------------------------------------------------- score_tile on bf16 matrix cores

// fp32-accurate products on the bf16 matrix cores (16x the fp32 MFMA rate on gfx950):
// each fp32 operand x is split into three bf16 parts, x = x1 + x2 + x3 up to 2^-27
// relative (x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2); the differences
// are exact in fp32), and a.b is the sum of the six partial products whose part
// indices add to at most 4 (the dropped ones are below 2^-23 of |a b|), each exact in
// fp32 and summed by the MFMA in fp32: the error is of the order of an fp32 dot
// product's rounding.
__device__ __forceinline__ void split3_bf16(float x, __bf16 &h, __bf16 &m, __bf16 &l)
{
    h = (__bf16)x;
    const float r1 = x - (float)h;
    m = (__bf16)r1;
    l = (__bf16)(r1 - (float)m);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Pooled fp32 keys, d = 128, 512 threads: 128 rows x 64 candidates per tile, 8
// wavefronts in 4 x 2, each a 32 x 32 block of 2 x 2 MFMA 16x16x32 bf16 tiles.  The
// selector rows' three bf16 planes stay in registers; each staged key tile is split
// into three bf16 planes once, as it is written to LDS (two buffers, one barrier per
// tile).  Same output (order keys, group maxima) and layout as score_tile_kernel.
constexpr int kSplitPitch = 272;                         // bytes per 128-element bf16 plane row
constexpr int kSplitPlane = 64 * kSplitPitch;

__global__ __launch_bounds__(512, 1) void score_tile3_kernel(KP P, const uint16_t *__restrict__ q,
                                                             const float *__restrict__ kbase,
                                                             uint32_t *__restrict__ ws, long long stride,
                                                             int col_tiles, uint32_t *__restrict__ gmax,
                                                             long long gstride)
{
    constexpr int D = 128, NT = 512, KS = D / 32;
    constexpr int kPieces = 64 * D / 4 / NT;              // 16-byte fp32 pieces per thread per tile: 4
    __shared__ __attribute__((aligned(16))) unsigned char sh_k[2][3 * kSplitPlane];
    const int b = blockIdx.z % P.batch, c = blockIdx.z / P.batch;
    const Seq s = seq_info(P, b);
    const int r0 = blockIdx.y * 128;
    if (r0 >= s.n_q)
        return;
    const int r_end = min(r0 + 128, s.n_q);
    int jlo_last, jhi_last;
    row_cands(P, s.n_k, s.q0 + r_end - 1, jlo_last, jhi_last);
    jhi_last = min(jhi_last, (int)stride);
    const int jc_base = jlo_last;
    const int jc0 = jc_base + blockIdx.x * col_tiles * 64;
    if (jc0 >= jhi_last)
        return;
    const int jc1 = min(jc0 + col_tiles * 64, jhi_last);
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int li = lane % 16, lk = lane / 16;
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;

    // selector operands: rows r0 + wr + 16a + li, elements 32ks + 8lk .. +8, three planes
    bf16x8_t qa[2][KS][3];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        const int rl = r0 + wr + 16 * a + li;
        float qs[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                qs[ks][e] = 0.f;
        if (rl < r_end) {
            const long long i = s.q_off + rl;
            for (int h = 0; h < P.G; h++) {
                const uint16_t *qp = q + (i * P.h_q + (long long)c * P.G + h) * D + 8 * lk;
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(qp + 32 * ks);
                    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        qs[ks][2 * e] += __uint_as_float(wd[e] << 16);
                        qs[ks][2 * e + 1] += __uint_as_float(wd[e] & 0xffff0000u);
                    }
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int e = 0; e < 8; e++) {
                __bf16 h, m, l;
                split3_bf16(qs[ks][e], h, m, l);
                qa[a][ks][0][e] = h;
                qa[a][ks][1][e] = m;
                qa[a][ks][2][e] = l;
            }
    }
    // the products come out transposed (candidates down, rows across): lane (li, lk)
    // holds four consecutive candidates 4 lk .. +3 of row li of each 16 x 16 tile
    int jh_row[2];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        const int rl = r0 + wr + 16 * a + li;
        int jl = 0, jh = 0;
        if (rl < r_end)
            row_cands(P, s.n_k, s.q0 + rl, jl, jh);
        jh_row[a] = jh > jl ? min(jh, (int)stride) : 0;
    }
    const int j_first = first_cand(P);
    const float *kb0 = kbase + (((long long)c * P.batch + b) * P.nb_max) * D;
    // staging: thread tid holds fp32 pieces tid + NT u (row = piece / 32, 4 elements at 4 (piece % 32))
    float4 stage[kPieces];
    auto issue = [&](int jt) {
#pragma unroll
        for (int u = 0; u < kPieces; u++) {
            const int piece = tid + NT * u, row = piece >> 5, col = piece & 31;
            const int j = min(jt + row, jhi_last - 1);       // rows past the end re-read the last one
            stage[u] = *reinterpret_cast<const float4 *>(kb0 + (long long)j * D + 4 * col);
        }
    };
    auto write = [&](unsigned char *buf) {
#pragma unroll
        for (int u = 0; u < kPieces; u++) {
            const int piece = tid + NT * u, row = piece >> 5, col = piece & 31;
            const float x[4] = {stage[u].x, stage[u].y, stage[u].z, stage[u].w};
            bf16x4_t ph, pm, pl;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                __bf16 h, m, l;
                split3_bf16(x[e], h, m, l);
                ph[e] = h;
                pm[e] = m;
                pl[e] = l;
            }
            unsigned char *dst = buf + row * kSplitPitch + 8 * col;
            *reinterpret_cast<bf16x4_t *>(dst) = ph;
            *reinterpret_cast<bf16x4_t *>(dst + kSplitPlane) = pm;
            *reinterpret_cast<bf16x4_t *>(dst + 2 * kSplitPlane) = pl;
        }
    };
    auto tile = [&](const unsigned char *buf, int jt) {
        floatx4 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int bb = 0; bb < 2; bb++)
                acc[a][bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            bf16x8_t kv[2][3];
#pragma unroll
            for (int bb = 0; bb < 2; bb++)
#pragma unroll
                for (int pl = 0; pl < 3; pl++)
                    kv[bb][pl] = *reinterpret_cast<const bf16x8_t *>(buf + pl * kSplitPlane +
                                                                     (wc + 16 * bb + li) * kSplitPitch + 64 * ks +
                                                                     16 * lk);
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int bb = 0; bb < 2; bb++) {
                    // S^T = K Q^T (keys as the A operand); smallest terms first:
                    // (3,1), (2,2), (1,3), (2,1), (1,2), (1,1)
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][0], qa[a][ks][2], acc[a][bb], 0, 0, 0);
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][1], qa[a][ks][1], acc[a][bb], 0, 0, 0);
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][2], qa[a][ks][0], acc[a][bb], 0, 0, 0);
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][0], qa[a][ks][1], acc[a][bb], 0, 0, 0);
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][1], qa[a][ks][0], acc[a][bb], 0, 0, 0);
                    acc[a][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[bb][0], qa[a][ks][0], acc[a][bb], 0, 0, 0);
                }
        }
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const int rl = r0 + wr + 16 * a + li;
            uint32_t *dst = ws + ((long long)c * P.rows + s.q_off + rl) * stride + key_col0(P);
            uint32_t m = 0u;
#pragma unroll
            for (int bb = 0; bb < 2; bb++) {
                // candidates j0 .. j0+3: key_col0 + j0 is a multiple of 4 (the span starts at
                // the first candidate), so four valid keys are one 16-byte store
                const int j0 = jt + wc + 16 * bb + 4 * lk;
                uint32_t kk[4];
                bool ok[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    kk[i] = order_key(acc[a][bb][i]);
                    ok[i] = j0 + i >= j_first && j0 + i < jh_row[a];
                    m = max(m, ok[i] ? kk[i] : 0u);
                }
                if (ok[0] && ok[3]) {                     // the valid candidates are one range
                    *reinterpret_cast<uint4 *>(dst + j0) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (ok[i])
                            dst[j0 + i] = kk[i];
                }
            }
            // the wavefront's 32 columns of row li are one group: its lanes li, li+16, li+32, li+48
            m = max(m, (uint32_t)__shfl_xor((int)m, 16, kWave));
            m = max(m, (uint32_t)__shfl_xor((int)m, 32, kWave));
            if (gmax && lk == 0 && rl < r_end && jt + wc < jc1)
                gmax[((long long)c * P.rows + s.q_off + rl) * gstride + (unsigned)(jt + wc - jc_base) / kGroupCols] = m;
        }
    };
    const int n_t = (jc1 - jc0 + 63) / 64;
    issue(jc0);
    write(sh_k[0]);
    issue(jc0 + 64);
    for (int t = 0; t < n_t; t++) {
        __syncthreads();                                  // buffer t&1 holds tile t
        tile(sh_k[t & 1], jc0 + 64 * t);
        write(sh_k[(t + 1) & 1]);
        issue(jc0 + 64 * (t + 2));
    }
}

// ---------------------------------------------------------------- top-k over the workspace

// One row's selection by one wavefront, its keys held K per lane.
template <int K>
__device__ __forceinline__ void topk_wave_row(const uint32_t *src, const RowGeo &r, int32_t *out, uint32_t *sk,
                                              int *si)
{
    const int lane = lane_id();
    uint32_t kr[K];
#pragma unroll
    for (int m = 0; m < K; m++) {
        const int i = m * kWave + lane;
        kr[m] = i < r.n_cand ? src[r.j_lo + i] : 0u;
    }
    wave_select<K>(kr, r.n_cand, r.need, EmitIdx{out, r.j_lo}, sk, si);
}

// 4 wavefronts per workgroup, one row each (<= 64 * KPL candidates).  grid: (ceil(rows/4), h_kv).
// A row takes the smallest keys-per-lane count that holds it, so a wavefront's work
// follows its row's length (the rows of a causal prefill range from none to the stride).
template <int KPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(KP P, const uint32_t *__restrict__ ws,
                                                        long long stride, int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ n_idx)
{
    const long long row = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    const int c = blockIdx.y, lane = lane_id();
    if (row >= P.rows)
        return;
    // only the row's own candidates are read (a causal row of a prefill holds fewer than
    // the stride: on average half of it)
    RowGeo r = row_geo(P, row);
    const uint32_t *src = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (lane == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, lane, kWave);
        return;
    }
    __shared__ uint32_t sh_k[4][kFilterCap];
    __shared__ int sh_i[4][kFilterCap];
    const int wv = threadIdx.x / kWave;
    if (KPL > 4 && r.n_cand <= 4 * kWave)
        topk_wave_row<(KPL > 4 ? 4 : KPL)>(src, r, out, sh_k[wv], sh_i[wv]);
    else if (KPL > 8 && r.n_cand <= 8 * kWave)
        topk_wave_row<(KPL > 8 ? 8 : KPL)>(src, r, out, sh_k[wv], sh_i[wv]);
    else if (KPL > 16 && r.n_cand <= 16 * kWave)
        topk_wave_row<(KPL > 16 ? 16 : KPL)>(src, r, out, sh_k[wv], sh_i[wv]);
    else
        topk_wave_row<KPL>(src, r, out, sh_k[wv], sh_i[wv]);
    for (int s = r.need + lane; s < P.topk; s += kWave)
        out[s] = -1;
}

// Exclusive block-wide scan of one int per thread (NT threads); returns (exclusive, total).
template <int NT>
__device__ __forceinline__ int2 block_scan_int(int v, int *sh)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
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
    for (int i = 0; i < NT / kWave; i++) {
        int c = sh[i];
        off += i < w ? c : 0;
        tot += c;
    }
    __syncthreads();
    return make_int2(off + incl - v, tot);
}

constexpr int kCompactMaxN = 262144;     // candidates per row (bitmap of 8192 words in LDS)
constexpr int kCompactCap = 4032;        // keys kept for the exact last step (LDS of two workgroups per CU)

// Calls f(i, key) for every key i in [0, n) of a row whose keys start at element
// j_lo of a 16-byte aligned row base: 16-byte loads, eight per thread in flight.
template <int NT, typename F>
__device__ __forceinline__ void for_each_key(const uint32_t *row, int j_lo, int n, F f)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(row);
    const int q_lo = j_lo >> 2, q_hi = (j_lo + n + 3) >> 2;
    constexpr int U = 8;
    for (int q0 = q_lo + (int)threadIdx.x; q0 < q_hi; q0 += NT * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int q = q0 + u * NT;
            v[u] = q < q_hi ? p[q] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int q = q0 + u * NT;
            const uint32_t e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int i = 4 * q + e - j_lo;
                if (q < q_hi && i >= 0 && i < n)
                    f(i, e4[e]);
            }
        }
    }
}

// One 1024-thread workgroup per row, 2048 < candidates <= 262144.
//  0. for k <= 512 and rows of >= 65536 keys: gather the keys >= the k-th largest
//     per-thread maximum (below);
//     otherwise, or when more than kCompactCap keys pass:
//  1. histograms of 12, 12 and 8 key bits (most significant first), each restricted to
//     the prefix chosen so far, until the bin holding the k-th largest key has at most
//     kCompactCap keys (usually after the first histogram: the selected tail is thin);
//  2. one pass marks every key above that bin in an LDS bitmap and copies the bin's
//     keys and indices to LDS;
//  3. the remaining picks are made exactly inside LDS (binary search on the key, then
//     on the index for equal keys: ties go to the lower index);
//  4. the bitmap is compacted into ascending indices.
// The keys are read from the workspace two to four times in all.  With the group
// maxima of the scoring (gmax, rows of >= 4k groups of 32 keys), step 0 instead
// takes t0 = a value that k group maxima reach and reads only the groups whose
// maximum reaches it (about k of them, k x 128 bytes instead of the whole row).
// Two workgroups per CU (8 wavefronts per SIMD): the launch bounds keep the SGPRs at or
// below the 100 that allows (102 without them held it to 7, one workgroup per CU).
__global__ __launch_bounds__(1024, 8) void topk_compact_kernel(KP P, const uint32_t *__restrict__ ws, long long stride,
                                                            int32_t *__restrict__ idx, int32_t *__restrict__ n_idx,
                                                            const uint32_t *__restrict__ gmax, long long gstride)
{
    constexpr int NT = 1024, NW = NT / kWave;
    __shared__ int hist[4096];
    __shared__ uint32_t bitmap[kCompactMaxN / 32];
    __shared__ uint32_t cand_key[kCompactCap];
    __shared__ int cand_idx[kCompactCap];
    __shared__ int sh_scan[NW];
    __shared__ int sh_digit, sh_above, sh_ncand;
    __shared__ int sh_cnt3[3];
    __shared__ int sh_cnt16[2][16];
    const long long row = blockIdx.x;
    const int c = blockIdx.y, tid = threadIdx.x, lane = lane_id();
    RowGeo r = row_geo(P, row);
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    if (tid == 0)
        n_idx[(long long)c * P.rows + row] = r.need;
    if (r.need == r.n_cand) {
        write_all(P, out, r, tid, NT);
        return;
    }
    const int n = min(r.n_cand, kCompactMaxN);
    const int need = min(r.need, n);
    if (need == 0) {
        for (int s2 = tid; s2 < P.topk; s2 += NT)
            out[s2] = -1;
        return;
    }
    const uint32_t *row_keys = ws + ((long long)c * P.rows + row) * stride;   // 128-byte aligned
    const int j_lo = r.j_lo + key_col0(P);                  // the row's first candidate in row_keys
    const uint32_t *keys = row_keys + j_lo;
    const int nword = (n + 31) / 32;
    for (int x = tid; x < nword; x += NT)
        bitmap[x] = 0u;
    uint32_t prefix = 0, pmask = 0;
    int rem = need;
    bool gather = false;
    // Block-wide counts at one barrier each: wavefront ballots summed by LDS atomics
    // into one of three rotating counters (the one two rounds ahead is cleared once
    // every thread has read the last round's).
    if (tid < 3)
        sh_cnt3[tid] = 0;
    __syncthreads();
    int rnd = 0;
    auto block_total = [&](int wave_cnt) -> int {        // wave_cnt: uniform across the wavefront
        if (lane == 0 && wave_cnt)
            atomicAdd(&sh_cnt3[rnd % 3], wave_cnt);
        __syncthreads();
        const int tot = sh_cnt3[rnd % 3];
        if (tid == 0)
            sh_cnt3[(rnd + 2) % 3] = 0;
        rnd++;
        return tot;
    };
    const int ng = (n + kGroupCols - 1) / kGroupCols;
    if (gmax && need <= NT / 2 && ng >= 4 * need) {
        // Thread tid owns the gpt consecutive groups from gpt * tid, so at least
        // min(ng, 513) >= need threads own one.  t0 = the need-th largest of the threads'
        // maxima over their groups: need keys reach it, so the need-th largest key does
        // and every selected key is >= t0.  Only the groups whose maximum reaches t0
        // are read.  ng <= 8192.
        const uint32_t *gm_row = gmax + ((long long)c * P.rows + row) * gstride;
        const int gpt = (ng + NT - 1) / NT;
        uint32_t gm[kCompactMaxN / kGroupCols / NT];
        uint32_t tm = 0u;
#pragma unroll
        for (int m = 0; m < kCompactMaxN / kGroupCols / NT; m++) {
            const int x = gpt * tid + m;
            gm[m] = m < gpt && x < ng ? gm_row[x] : 0u;
            tm = max(tm, gm[m]);
        }
        hist[tid] = (int)tm;
        __syncthreads();
        uint32_t kr[NT / kWave];
#pragma unroll
        for (int m = 0; m < NT / kWave; m++)
            kr[m] = (uint32_t)hist[m * kWave + lane];
        const uint32_t t0 = block_threshold16<NT / kWave>(kr, NT, need, 0u, 28, sh_cnt16);
        // the groups reaching t0, listed in ascending order (in hist)
        int f = 0;
#pragma unroll
        for (int m = 0; m < kCompactMaxN / kGroupCols / NT; m++)
            f += m < gpt && gpt * tid + m < ng && gm[m] >= t0 ? 1 : 0;
        const int2 sc = block_scan_int<NT>(f, sh_scan);       // its barriers also retire the reads of hist
        const int n_grp = sc.y;
        if (n_grp <= 4096) {
            int o = sc.x;
#pragma unroll
            for (int m = 0; m < kCompactMaxN / kGroupCols / NT; m++)
                if (m < gpt && gpt * tid + m < ng && gm[m] >= t0)
                    hist[o++] = gpt * tid + m;
        }
        if (tid == 0)
            sh_ncand = 0;
        __syncthreads();
        if (n_grp <= 4096) {
            // their keys >= t0 into cand_key / cand_idx (one LDS atomic per wavefront and round)
            const uint32_t *keys = row_keys + j_lo;
            const int tot = n_grp * kGroupCols;
            constexpr int U = 16;
            for (int e0 = 0; e0 < tot; e0 += NT * U) {
                uint32_t kv[U];
                int iv[U];
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int e = e0 + u * NT + tid;
                    iv[u] = e < tot ? hist[e / kGroupCols] * kGroupCols + e % kGroupCols : n;
                    kv[u] = iv[u] < n ? keys[iv[u]] : 0u;
                }
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const bool take = iv[u] < n && kv[u] >= t0;
                    const unsigned long long mk = __ballot(take);
                    if (mk) {
                        int base = 0;
                        if (lane == 0)
                            base = atomicAdd(&sh_ncand, __popcll(mk));
                        base = __builtin_amdgcn_readfirstlane(base);
                        const int slot = base + lanes_below(mk);
                        if (take && slot < kCompactCap) {
                            cand_key[slot] = kv[u];
                            cand_idx[slot] = iv[u];
                        }
                    }
                }
            }
        }
        __syncthreads();
        gather = n_grp <= 4096 && sh_ncand <= kCompactCap;
        __syncthreads();
    } else if (need <= NT / 2 && n >= 65536) {
        // Long rows (its 32 block-wide counting rounds cost more than a histogram on
        // short ones).  Threshold from the per-thread maxima: at least min(n, NT) >= need threads hold
        // keys, so at least `need` keys are >= t0 = the need-th largest thread maximum
        // and every selected key is >= t0 (threads without keys keep 0, below every
        // key).  One pass of maxima, one pass gathering the keys >= t0 (about 0.3% of
        // the row for need = 512 of 262144) -- no histogram atomics on the crowded
        // exponent bins.  More than kCompactCap such keys fall back to the histograms.
        uint32_t mx = 0u;
        for_each_key<NT>(row_keys, j_lo, n, [&](int, uint32_t k) { mx = max(mx, k); });
        uint32_t t0 = 0u;                                  // a threshold that need maxima reach
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = t0 | (1u << bit);
            const int cnt = block_total(__popcll(__ballot(mx >= cand)));
            if (cnt >= need)
                t0 = cand;
            if (cnt == need)
                break;
        }
        if (tid == 0)
            sh_ncand = 0;
        __syncthreads();
        for_each_key<NT>(row_keys, j_lo, n, [&](int i, uint32_t k) {
            if (k >= t0) {
                const int slot = atomicAdd(&sh_ncand, 1);
                if (slot < kCompactCap) {
                    cand_key[slot] = k;
                    cand_idx[slot] = i;
                }
            }
        });
        __syncthreads();
        gather = sh_ncand <= kCompactCap;
        __syncthreads();
    }
    if (!gather) {
        int cnt_bin = 0;
        const int shifts[3] = {20, 8, 0};
        const int widths[3] = {12, 12, 8};
        for (int level = 0; level < 3; level++) {
            const int shift = shifts[level], nb = 1 << widths[level];
            for (int x = tid; x < nb; x += NT)
                hist[x] = 0;
            __syncthreads();
            for_each_key<NT>(row_keys, j_lo, n, [&](int, uint32_t k) {
                if ((k & pmask) == prefix)
                    atomicAdd(&hist[(k >> shift) & (nb - 1)], 1);
            });
            __syncthreads();
            // digit holding the rem-th largest key: scan the bins from the top
            const int per = nb / NT > 0 ? nb / NT : 1;           // bins per thread (4 or 1)
            int loc = 0;
            const int b0 = nb - 1 - tid * per;                   // this thread's bins: b0, b0-1, ...
            for (int q = 0; q < per; q++)
                if (tid * per + q < nb)
                    loc += hist[b0 - q];
            int2 sc = block_scan_int<NT>(tid * per < nb ? loc : 0, sh_scan);
            if (tid * per < nb && sc.x < rem && sc.x + loc >= rem) {
                int run = sc.x;
                for (int q = 0; q < per; q++) {
                    int h = hist[b0 - q];
                    if (run + h >= rem) {
                        sh_digit = b0 - q;
                        sh_above = run;
                        break;
                    }
                    run += h;
                }
            }
            __syncthreads();
            const int d = sh_digit;
            prefix |= ((uint32_t)d) << shift;
            pmask |= ((uint32_t)(nb - 1)) << shift;
            rem -= sh_above;
            cnt_bin = hist[d];
            __syncthreads();
            if (cnt_bin <= kCompactCap)
                break;
        }
        // mark keys above the bin, gather the bin
        if (tid == 0)
            sh_ncand = 0;
        __syncthreads();
        const uint32_t top_of_bin = prefix | ~pmask;
        gather = cnt_bin <= kCompactCap;
        for_each_key<NT>(row_keys, j_lo, n, [&](int i, uint32_t k) {
            if (k > top_of_bin) {
                atomicOr(&bitmap[i >> 5], 1u << (i & 31));
            } else if (gather && (k & pmask) == prefix) {
                int slot = atomicAdd(&sh_ncand, 1);
                cand_key[slot] = k;
                cand_idx[slot] = i;
            }
        });
        __syncthreads();
    }
    if (gather) {
        // exact pick of rem among the gathered keys: tau = rem-th largest key
        const int nc = sh_ncand;
        auto block_count = [&](auto pred) -> int {
            int cnt = 0;
            for (int base = 0; base < nc; base += NT) {
                const int x = base + tid;
                cnt += __popcll(__ballot(x < nc && pred(x)));
            }
            return block_total(cnt);
        };
        uint32_t tau = prefix;
        int n_gt, n_eq;
        const int free_bits = 32 - __popc(pmask);              // the prefix fixes the top bits
        if (nc <= NT && free_bits % 4 == 0) {
            // every wavefront holds all gathered keys: 4 bits per round, then the counts
            // above and at tau without a barrier
            uint32_t kr[NT / kWave];
#pragma unroll
            for (int m = 0; m < NT / kWave; m++) {
                const int x = m * kWave + lane;
                kr[m] = x < nc ? cand_key[x] : 0u;
            }
            if (free_bits > 0)
                tau = block_threshold16<NT / kWave>(kr, nc, rem, prefix, free_bits - 4, sh_cnt16);
            n_gt = 0;
            n_eq = 0;
#pragma unroll
            for (int m = 0; m < NT / kWave; m++) {
                const bool valid = m * kWave + lane < nc;
                n_gt += __popcll(__ballot(valid && kr[m] > tau));
                n_eq += __popcll(__ballot(valid && kr[m] == tau));
            }
        } else {
            for (int bit = 31; bit >= 0; --bit) {
                if (pmask & (1u << bit))
                    continue;                                    // fixed by the prefix
                const uint32_t cand = tau | (1u << bit);
                const int cnt = block_count([&](int x) { return cand_key[x] >= cand; });
                if (cnt >= rem)
                    tau = cand;
                if (cnt == rem)                                  // exactly the selection: done
                    break;
            }
            n_gt = block_count([&](int x) { return cand_key[x] > tau; });
            n_eq = block_count([&](int x) { return cand_key[x] == tau; });
        }
        const int need_eq = rem - n_gt;
        // among keys == tau: the need_eq lowest indices (binary search on the index, skipped
        // when every equal key is taken -- the usual case of one)
        int ilim = 1 << 30;
        if (n_eq > need_eq) {
            int lo = 0;                                      // largest bound with count(idx < bound) <= need_eq
            for (int bit = 18; bit >= 0; --bit) {
                const int candb = lo | (1 << bit);
                if (block_count([&](int x) { return cand_key[x] == tau && cand_idx[x] < candb; }) <= need_eq)
                    lo = candb;
            }
            ilim = lo;
        }
        for (int x = tid; x < nc; x += NT) {
            const uint32_t k = cand_key[x];
            const int i = cand_idx[x];
            if (k > tau || (k == tau && i < ilim))
                atomicOr(&bitmap[i >> 5], 1u << (i & 31));
        }
    } else {
        // more than kCompactCap keys share the full 32-bit key: the lowest indices win
        int seen = 0;
        for (int base = 0; base < n; base += NT) {
            const int i = base + tid;
            const bool eq = i < n && keys[i] == prefix;
            int2 e = block_scan_int<NT>(eq ? 1 : 0, sh_scan);
            if (eq && seen + e.x < rem)
                atomicOr(&bitmap[i >> 5], 1u << (i & 31));
            seen += e.y;
        }
    }
    __syncthreads();
    // ascending output from the bitmap
    const int wpt = (nword + NT - 1) / NT;                    // words per thread
    int cnt = 0;
    for (int q = 0; q < wpt; q++) {
        int wd = tid * wpt + q;
        cnt += wd < nword ? __popc(bitmap[wd]) : 0;
    }
    int pos = block_scan_int<NT>(cnt, sh_scan).x;
    for (int q = 0; q < wpt; q++) {
        int wd = tid * wpt + q;
        uint32_t bits = wd < nword ? bitmap[wd] : 0u;
        while (bits) {
            int bpos = __ffs(bits) - 1;
            bits &= bits - 1;
            if (pos < P.topk)
                out[pos] = r.j_lo + wd * 32 + bpos;
            pos++;
        }
    }
    for (int s2 = need + tid; s2 < P.topk; s2 += NT)
        out[s2] = -1;
    (void)lane;
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
    if (r.need == r.n_cand || r.need == 0) {
        write_all(P, out, r.need == 0 ? RowGeo{r.b, r.n_k, r.p_sel, r.q_first, r.q_last, r.j_lo, r.j_lo, 0, 0, r.k_off}
                                      : r, threadIdx.x, NT);
        return;
    }
    block_topk<NT>(ws + ((long long)c * P.rows + row) * stride + key_col0(P) + r.j_lo, r.n_cand, r.need, r.j_lo,
                   out);
    for (int s = r.need + (int)threadIdx.x; s < P.topk; s += NT)
        out[s] = -1;
}

// Every row: n_idx = 0 and no index (k = 0 everywhere).
__global__ void select_empty_kernel(KP P, int32_t *__restrict__ n_idx)
{
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < P.rows * P.h_kv) {
        n_idx[i] = 0;
        if (P.boundary)
            boundary_none(P, i % P.rows, (int)(i / P.rows));
    }
}

// Boundary scores of the plans that keep every candidate's key in the workspace: one
// workgroup per (row, KV head) reads the row's keys and its selection (ascending,
// kept in LDS when it fits, else searched in place) and reduces the smallest selected
// and the largest unselected key.  Runs after the top-k, only for the audit.
constexpr int kBoundarySel = 4096;

__global__ __launch_bounds__(256) void boundary_ws_kernel(KP P, const uint32_t *__restrict__ ws, long long stride,
                                                          const int32_t *__restrict__ idx)
{
    __shared__ int sh_sel[kBoundarySel];
    __shared__ uint32_t sh_red[2][4];
    const long long row = blockIdx.x;
    const int c = blockIdx.y, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const RowGeo r = row_geo(P, row);
    if (r.need == 0 || r.need == r.n_cand) {
        if (tid == 0)
            boundary_none(P, row, c);
        return;
    }
    const int32_t *sel_g = idx + ((long long)c * P.rows + row) * P.topk;
    const bool in_lds = r.need <= kBoundarySel;
    if (in_lds)
        for (int x = tid; x < r.need; x += 256)
            sh_sel[x] = sel_g[x];
    __syncthreads();
    const int32_t *sel = in_lds ? sh_sel : sel_g;
    const uint32_t *src = ws + ((long long)c * P.rows + row) * stride + key_col0(P);
    uint32_t kept = 0xffffffffu, left = 0u;
    for (int i = tid; i < r.n_cand; i += 256) {
        const int j = r.j_lo + i;
        const uint32_t key = src[j];
        int lo = 0, hi = r.need;                          // first selected index >= j
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sel[mid] < j)
                lo = mid + 1;
            else
                hi = mid;
        }
        if (lo < r.need && sel[lo] == j)
            kept = min(kept, key);
        else
            left = max(left, key);
    }
    kept = wave_min_u32(kept);
    left = wave_max_u32(left);
    if (lane == 0) {
        sh_red[0][w] = kept;
        sh_red[1][w] = left;
    }
    __syncthreads();
    if (tid == 0)
        boundary_store(P, row, c, min(min(sh_red[0][0], sh_red[0][1]), min(sh_red[0][2], sh_red[0][3])),
                       max(max(sh_red[1][0], sh_red[1][1]), max(sh_red[1][2], sh_red[1][3])));
}

// ---------------------------------------------------------------- dispatch

static constexpr int kWaveTopkMax = 2048;
static constexpr int kSplitChunk = 512;  // candidates per scoring workgroup (a multiple of every round size)

// Candidate capacity of a row, and the row pitch of the score-key workspace (a
// multiple of 32 with room for the key_col0 shift, so every row starts a 128-byte
// line).
static constexpr long long kRowFusedMin = 256;          // rows x KV heads for the fused row plan

static long long cand_cap(const KP &P) { return P.g == 1 ? P.max_k : P.nb_max; }
static long long key_stride(const KP &P) { return (cand_cap(P) + 31) / 32 * 32 + 32; }

// Group maxima of the scores (tile scoring followed by the compacting top-k): their
// row stride, or 0 when not kept.
static long long gmax_stride(const KP &P, int plan)
{
    const long long cap = cand_cap(P);
    if (plan != kSelectTile || cap <= kWaveTopkMax || cap > kCompactMaxN || getenv("SPARSE_ATTN_TOPK_RADIX"))
        return 0;
    return ((cap + kGroupCols - 1) / kGroupCols + 3) / 4 * 4;
}

size_t select_workspace_bytes(const KP &P, int plan)
{
    if (plan == kSelectEmpty || plan == kSelectRowFused)
        return 0;
    if (plan == kSelectHeads) {                           // order keys, and every head's logits for SOFTMAX
        const size_t per = (size_t)P.h_kv * (size_t)P.rows * (size_t)key_stride(P) * sizeof(uint32_t);
        return per * (P.select_mode == 1 ? 1 + (size_t)P.G : 1);
    }
    const long long stride = plan == kSelectRow ? cand_cap(P) : key_stride(P);
    if (plan == kSelectRow) {                             // (key, position) survivors of every part
        const long long n_part = (stride + kPartCand - 1) / kPartCand;
        return (size_t)P.h_kv * (size_t)P.rows * (size_t)n_part * (size_t)part_cap(P.topk) * 2 * sizeof(uint32_t);
    }
    return (size_t)P.h_kv * (size_t)P.rows * (size_t)(stride + gmax_stride(P, plan)) * sizeof(uint32_t);
}

int select_plan(const KP &P)
{
    if (P.topk == 0)
        return kSelectEmpty;
    if (P.select_mode != 0)
        return kSelectHeads;
    bool few_rows = P.shared || P.max_q <= 8;
    long long max_cand = P.g == 1 ? P.max_k : P.nb_max;
    // one workgroup per (row, KV head) once that gives every CU one; parts + merge below
    const int row_plan = P.rows * P.h_kv >= kRowFusedMin ? kSelectRowFused : kSelectRow;
    int plan = !few_rows ? kSelectTile : (max_cand <= kRowMaxCand ? row_plan : kSelectSplit);
    if (const char *e = getenv("SPARSE_ATTN_SELECT_PLAN")) {       // tuning override
        int v = atoi(e);
        if (few_rows && (v == kSelectSplit || ((v == kSelectRow || v == kSelectRowFused) && max_cand <= kRowMaxCand)))
            plan = v;
    }
    return plan;
}

template <typename T, int D>
static hipError_t launch_select_t(const KP &P, const void *q_sel, const float *k_cmp, const void *k,
                                  int32_t *idx, int32_t *n_idx, void *ws, hipEvent_t ev0, hipEvent_t ev1,
                                  hipStream_t st, const SelAppend &app)
{
    // the optional event pair brackets the scoring kernel (the one that reads the keys)
    const bool timed = ev0 && ev1;
    auto mark = [&](hipEvent_t ev) {
        if (timed)
            (void)hipEventRecord(ev, st);
    };
    const T *q = (const T *)q_sel;
    int plan = select_plan(P);
    const long long stride = plan == kSelectRow ? cand_cap(P) : key_stride(P);
    uint32_t *wsk = (uint32_t *)ws;
    const long long gms = gmax_stride(P, plan);
    uint32_t *gm = gms ? wsk + (size_t)P.h_kv * (size_t)P.rows * (size_t)stride : nullptr;
    if (plan == kSelectEmpty) {
        long long n = P.rows * P.h_kv;
        select_empty_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(P, n_idx);
        return hipGetLastError();
    }
    if (plan == kSelectRowFused) {
        dim3 grid((unsigned)(P.rows * P.h_kv));
        mark(ev0);
        if (P.g == 1)
            select_row_kernel<T, T, D><<<grid, dim3(1024), 0, st>>>(P, q, (const T *)k, idx, n_idx, app);
        else
            select_row_kernel<T, float, D><<<grid, dim3(1024), 0, st>>>(P, q, k_cmp, idx, n_idx, app);
        mark(ev1);
        return hipGetLastError();
    }
    if (plan == kSelectRow) {
        const int n_part = (int)((stride + kPartCand - 1) / kPartCand);
        const size_t n_slot = (size_t)P.h_kv * (size_t)P.rows * (size_t)n_part * (size_t)part_cap(P.topk);
        uint32_t *ws_k = wsk;
        int32_t *ws_i = (int32_t *)(wsk + n_slot);
        dim3 grid((unsigned)(P.rows * n_part), (unsigned)P.h_kv);
        mark(ev0);
        if (P.g == 1)
            select_part_kernel<T, T, D><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, ws_k, ws_i, n_part);
        else
            select_part_kernel<T, float, D><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, ws_k, ws_i, n_part);
        mark(ev1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        // survivors per row <= n_part * min(need, kPartCand) <= the row's candidates
        const long long m_max = (long long)n_part * part_cap(P.topk) < stride ? (long long)n_part * part_cap(P.topk)
                                                                             : stride;
        dim3 mgrid((unsigned)((P.rows + 3) / 4), (unsigned)P.h_kv);
        if (m_max <= 128)
            select_merge_kernel<2><<<mgrid, dim3(256), 0, st>>>(P, ws_k, ws_i, n_part, idx, n_idx);
        else if (m_max <= 256)
            select_merge_kernel<4><<<mgrid, dim3(256), 0, st>>>(P, ws_k, ws_i, n_part, idx, n_idx);
        else if (m_max <= 512)
            select_merge_kernel<8><<<mgrid, dim3(256), 0, st>>>(P, ws_k, ws_i, n_part, idx, n_idx);
        else
            select_merge_kernel<16><<<mgrid, dim3(256), 0, st>>>(P, ws_k, ws_i, n_part, idx, n_idx);
        return hipGetLastError();
    }
    mark(ev0);
    if (plan == kSelectHeads) {
        // 128-candidate chunks while the grid would hold fewer than 1024 workgroups (decode)
        float *ws_l = reinterpret_cast<float *>(wsk + (size_t)P.h_kv * (size_t)P.rows * (size_t)stride);
        const bool small = P.rows * P.h_kv * ((stride + kSplitChunk - 1) / kSplitChunk) < 1024;
        const int ch = small ? 128 : kSplitChunk;
        const int n_chunk = (int)((stride + ch - 1) / ch);
        dim3 grid((unsigned)(P.rows * n_chunk), (unsigned)P.h_kv);
        if (P.select_mode == 3) {
            // bf16 token keys and rows of <= 16 (query, head) pairs: the matrix-core scorer
            const bool mma = sizeof(T) == 2 && D == 128 && P.g == 1 &&
                             (long long)(P.shared ? P.max_q : 1) * P.G <= 16 && !getenv("SPARSE_ATTN_ATTN_VALU");
            if (mma && small)
                score_attn_mfma_kernel<128><<<grid, dim3(256), 0, st>>>(P, (const uint16_t *)q, (const uint16_t *)k,
                                                                      wsk, stride, n_chunk);
            else if (mma)
                score_attn_mfma_kernel<kSplitChunk><<<grid, dim3(256), 0, st>>>(P, (const uint16_t *)q,
                                                                              (const uint16_t *)k, wsk, stride,
                                                                              n_chunk);
            else if (small)
                score_attn_kernel<T, D, 128><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride, n_chunk);
            else
                score_attn_kernel<T, D, kSplitChunk><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride,
                                                                               n_chunk);
        } else if (P.g == 1) {
            if (small)
                score_heads_kernel<T, T, D, 128><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, ws_l, stride,
                                                                           n_chunk);
            else
                score_heads_kernel<T, T, D, kSplitChunk><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, ws_l,
                                                                                   stride, n_chunk);
        } else {
            if (small)
                score_heads_kernel<T, float, D, 128><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, ws_l, stride,
                                                                               n_chunk);
            else
                score_heads_kernel<T, float, D, kSplitChunk><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, ws_l,
                                                                                       stride, n_chunk);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (P.select_mode == 1)
            softmax_rows_kernel<<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(256), 0, st>>>(P, ws_l, wsk,
                                                                                              stride);
    } else if (plan == kSelectSplit) {
        int n_chunk = (int)((stride + kSplitChunk - 1) / kSplitChunk);
        dim3 grid((unsigned)(P.rows * n_chunk), (unsigned)P.h_kv);
        // One row per sequence, packed cache: the rows' candidates number at most
        // total_k / g + rows, so at most (total_k / g + rows) / CH + rows chunks; launch
        // those only (packed mapping) when that is fewer.
        if (P.shared && !P.block_table && P.rows <= 1024) {
            const long long bound = (P.total_k / P.g + P.rows) / kSplitChunk + P.rows + 1;
            if (bound < (long long)P.rows * n_chunk && !getenv("SPARSE_ATTN_SPLIT_GRID")) {
                grid.x = (unsigned)bound;
                n_chunk = 0;
            }
        }
        if (P.g == 1 && P.block_table)
            score_rows_kernel<T, T, D, kSplitChunk, 4><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride,
                                                                                 n_chunk);
        else if (P.g == 1 && n_chunk == 0)
            score_rows_kernel<T, T, D, kSplitChunk, 8, true><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk,
                                                                                       stride, n_chunk);
        else if (P.g == 1)
            score_rows_kernel<T, T, D, kSplitChunk, 8><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride,
                                                                                 n_chunk);
        else if (n_chunk == 0)
            score_rows_kernel<T, float, D, kSplitChunk, 8, true><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk,
                                                                                           stride, n_chunk);
        else
            score_rows_kernel<T, float, D, kSplitChunk, 8><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, stride,
                                                                                     n_chunk);
    } else {
        const bool split3 = P.g > 1 && sizeof(T) == 2 && D == 128 && !getenv("SPARSE_ATTN_SCORE_FP32");
        const int rt = split3 ? 128 : 64;                       // rows per workgroup
        const long long row_tiles = (long long)((P.max_q + rt - 1) / rt) * P.h_kv * P.batch;
        const int col_tiles = score_col_tiles(stride, row_tiles);
        dim3 grid((unsigned)((stride + col_tiles * 64 - 1) / (col_tiles * 64)), (unsigned)((P.max_q + rt - 1) / rt),
                  (unsigned)(P.h_kv * P.batch));
        if (split3)
            score_tile3_kernel<<<grid, dim3(512), 0, st>>>(P, (const uint16_t *)q, k_cmp, wsk, stride, col_tiles, gm,
                                                           gms);
        else if (P.g == 1)
            score_tile_kernel<T, T, D><<<grid, dim3(256), 0, st>>>(P, q, (const T *)k, wsk, stride, col_tiles, gm,
                                                                   gms);
        else
            score_tile_kernel<T, float, D><<<grid, dim3(256), 0, st>>>(P, q, k_cmp, wsk, stride, col_tiles, gm,
                                                                       gms);
    }
    mark(ev1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    dim3 tgrid((unsigned)((P.rows + 3) / 4), (unsigned)P.h_kv);
    const long long cap = cand_cap(P);                     // the top-k kernel by the candidates a row can hold
    if (cap <= 256)
        topk_wave_kernel<4><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (cap <= 512)
        topk_wave_kernel<8><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (cap <= 1024)
        topk_wave_kernel<16><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (cap <= kWaveTopkMax)
        topk_wave_kernel<32><<<tgrid, dim3(256), 0, st>>>(P, wsk, stride, idx, n_idx);
    else if (cap <= kCompactMaxN && !getenv("SPARSE_ATTN_TOPK_RADIX"))
        topk_compact_kernel<<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(1024), 0, st>>>(P, wsk, stride, idx,
                                                                                           n_idx, gm, gms);
    else
        topk_block_kernel<1024><<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(1024), 0, st>>>(
            P, wsk, stride, idx, n_idx);
    if (P.boundary) {
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        boundary_ws_kernel<<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(256), 0, st>>>(P, wsk, stride, idx);
    }
    return hipGetLastError();
}

static hipError_t launch_select_app(const KP &P, int dtype, const void *q_sel, const float *k_cmp, const void *k,
                                    int32_t *idx, int32_t *n_idx, void *ws, hipStream_t st, void *ev0, void *ev1,
                                    const SelAppend &app)
{
    hipEvent_t e0 = (hipEvent_t)ev0, e1 = (hipEvent_t)ev1;
    if (dtype == 1)
        return P.d == 128 ? launch_select_t<uint16_t, 128>(P, q_sel, k_cmp, k, idx, n_idx, ws, e0, e1, st, app)
                          : launch_select_t<uint16_t, 64>(P, q_sel, k_cmp, k, idx, n_idx, ws, e0, e1, st, app);
    return P.d == 128 ? launch_select_t<float, 128>(P, q_sel, k_cmp, k, idx, n_idx, ws, e0, e1, st, app)
                      : launch_select_t<float, 64>(P, q_sel, k_cmp, k, idx, n_idx, ws, e0, e1, st, app);
}

hipError_t launch_select(const KP &P, int dtype, const void *q_sel, const float *k_cmp, const void *k,
                         int32_t *idx, int32_t *n_idx, void *ws, hipStream_t st, void *ev0, void *ev1)
{
    return launch_select_app(P, dtype, q_sel, k_cmp, k, idx, n_idx, ws, st, ev0, ev1,
                             SelAppend{nullptr, nullptr, nullptr, nullptr, nullptr, 0});
}

// The append, then the selection.  Decode rows (one query per sequence, the row plan,
// pooled keys, window >= block so that no block the append re-pools is a candidate)
// run the append inside the selection's launch; otherwise two launches.
hipError_t launch_append_select(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                                float *k_cmp, const void *q_sel, int32_t *idx, int32_t *n_idx, void *ws,
                                hipStream_t st, void *ev0, void *ev1)
{
    const bool fused = k_cmp && P.g > 1 && !P.shared && P.max_q == 1 && P.window >= P.g && P.bucket_nb == 0 &&
                       select_plan(P) == kSelectRowFused;
    if (fused)
        return launch_select_app(P, dtype, q_sel, k_cmp, k, idx, n_idx, ws, st, ev0, ev1,
                                 SelAppend{k_new, v_new, k, v, k_cmp, append_pool_blocks(P)});
    hipError_t e = launch_append(P, dtype, k_new, v_new, k, v, k_cmp, st);
    if (e != hipSuccess)
        return e;
    return launch_select(P, dtype, q_sel, k_cmp, k, idx, n_idx, ws, st, ev0, ev1);
}

// The decode step in one launch (decode_step_kernel) when the step fits it: bf16 decode
// rows (one query per sequence) of the row plan with pooled keys and window >= block
// (the append's blocks are never candidates), the default group score, at most
// kStepRows heads per group, and an attended set that fits the LDS token list.
bool decode_step_fused_ok(const KP &P, int dtype, bool have_k_cmp)
{
    const long long a_max = (long long)P.n_init + (long long)P.topk * P.g + P.window;
    return dtype == 1 && have_k_cmp && P.g > 1 && !P.shared && P.max_q == 1 && P.window >= P.g &&
           P.select_mode == 0 && P.bucket_nb == 0 && P.G <= kStepRows && (P.d == 128 || P.d == 64) &&
           select_plan(P) == kSelectRowFused && a_max <= kTokCap && !getenv("SPARSE_ATTN_NO_STEP");
}

hipError_t launch_decode_step(const KP &P, int dtype, const void *k_new, const void *v_new, void *k, void *v,
                              float *k_cmp, const void *q, int32_t *idx, int32_t *n_idx, void *out, float *lse,
                              void *ws, int fwd_splits_n, hipStream_t st, void *ev0, void *ev1)
{
    if (!decode_step_fused_ok(P, dtype, k_cmp != nullptr)) {
        hipError_t e = launch_append_select(P, dtype, k_new, v_new, k, v, k_cmp, q, idx, n_idx, ws, st);
        if (e != hipSuccess)
            return e;
        return launch_fwd(P, dtype, q, k, v, idx, n_idx, out, lse, ws, fwd_splits_n, ev0, ev1, st);
    }
    const SelAppend app{k_new, v_new, k, v, k_cmp, append_pool_blocks(P)};
    dim3 grid((unsigned)(P.rows * P.h_kv));
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    if (P.d == 128)
        decode_step_kernel<128><<<grid, dim3(kStepWaves * 64), 0, st>>>(P, (const uint16_t *)q, k_cmp, (const uint16_t *)k,
                                                             (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
                                                             app);
    else
        decode_step_kernel<64><<<grid, dim3(kStepWaves * 64), 0, st>>>(P, (const uint16_t *)q, k_cmp, (const uint16_t *)k,
                                                            (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse,
                                                            app);
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev1, st);
    return hipGetLastError();
}

} // namespace sa
