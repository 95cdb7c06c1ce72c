// sa_common.hpp -- device-side helpers shared by the gfx950 kernels:
// kernel parameter block, sequence / selection geometry, element loads,
// wavefront reductions and the order-preserving score key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kWave = 64;

// Everything a kernel needs about the call, passed by value.
struct KP {
    int batch, h_q, h_kv, d, G;
    int max_q, max_k;
    long long total_q, total_k;
    const int32_t *cu_q, *cu_k, *q_pos0;
    int g, pool, topk;
    const int32_t *topk_per_seq;
    int n_init, window, shared;
    float scale_log2;   // softmax scale * log2(e): logits are kept in base 2
    float scale;        // softmax scale
    int nb_max;         // ceil(max_k / g)
    long long rows;     // selection rows per KV head
    int dtype;          // 0 fp32, 1 bf16
    const int32_t *block_table;   // paged K/V: [batch, max_pages] page ids, or nullptr (packed)
    int max_pages, page_shift;    // block-table row stride; log2(page_size)
    int pool_overlap;             // pooling window of block j starts at max(0, j*g - pool_overlap)
    int select_mode;              // 0 sum of heads, 1 sum of per-head softmaxes, 2 max over heads
    float head_score_scale;       // per-head score scale (1/tau or 1/sqrt(d))
    const float *attn_lse;        // select mode 3: [h_q, total_q] log-sum-exp of a dense verify pass
    // bucket selection (bucket_nb > 0): candidates are the buckets of the complete cluster
    // blocks of bucket_c tokens that end at or before p_sel, bucket_nb per block
    int bucket_c, bucket_nb, bucket_nblk;
    // optional selection audit: [h_kv, rows, 2] fp32, each row's need-th and (need+1)-th
    // scores (the smallest kept, the largest left out) times boundary_scale, or nullptr
    float *boundary;
    float boundary_scale;
    // contract-check word of this device (builds with SA_CHECKED), else nullptr
    uint32_t *check;
};

// Contract checks.  A build with SA_CHECKED defined validates what the kernels read
// from the caller's device tables: a gather whose index breaks the contract ORs its
// bit into *P.check and takes a clamped, in-range index instead.  Other builds
// compile every check away (the clamps they always apply stay).
enum : uint32_t {
    kCheckSeq = 1u,     // sequence geometry: cu_seqlens, lengths, q_pos0
    kCheckTable = 2u,   // selection table: an entry outside the row's blocks, or n_idx outside [0, topk]
    kCheckPage = 4u,    // block table: a negative page id
    kCheckToken = 8u    // a gathered token outside [0, p] of its query
};

__device__ __forceinline__ void contract_flag(uint32_t *word, bool bad, uint32_t bit)
{
#ifdef SA_CHECKED
    if (bad && word)
        atomicOr(word, bit);
#else
    (void)word;
    (void)bad;
    (void)bit;
#endif
}

struct Seq {
    long long k_off, q_off;
    int n_k, n_q, q0;
};

__device__ __forceinline__ Seq seq_info(const KP &P, int b)
{
    Seq s;
    s.k_off = P.cu_k[b];
    s.q_off = P.cu_q[b];
    s.n_k = P.cu_k[b + 1] - P.cu_k[b];
    s.n_q = P.cu_q[b + 1] - P.cu_q[b];
    s.q0 = P.q_pos0 ? P.q_pos0[b] : s.n_k - s.n_q;
#ifdef SA_CHECKED
    // offsets into [0, total], lengths into [0, max] and the rows' span, queries
    // inside their sequence
    const Seq r = s;
    s.k_off = s.k_off < 0 ? 0 : (s.k_off > P.total_k ? P.total_k : s.k_off);
    s.q_off = s.q_off < 0 ? 0 : (s.q_off > P.total_q ? P.total_q : s.q_off);
    const long long kmax = P.block_table ? (long long)P.max_k : min((long long)P.max_k, P.total_k - s.k_off);
    const long long qmax = min((long long)P.max_q, P.total_q - s.q_off);
    s.n_k = (int)(s.n_k < 0 ? 0 : (s.n_k > kmax ? kmax : s.n_k));
    s.n_q = (int)(s.n_q < 0 ? 0 : (s.n_q > qmax ? qmax : s.n_q));
    s.n_q = s.n_q > s.n_k ? s.n_k : s.n_q;
    s.q0 = s.q0 < 0 ? 0 : (s.q0 > s.n_k - s.n_q ? s.n_k - s.n_q : s.q0);
    contract_flag(P.check, r.k_off != s.k_off || r.q_off != s.q_off || r.n_k != s.n_k || r.n_q != s.n_q ||
                               r.q0 != s.q0, kCheckSeq);
#endif
    return s;
}

// Where token t of one sequence's K/V lives: row() is the token's row relative
// to kv_base() (the sequence's first row when packed, the pool's first row when
// paged: the block table read as a page table).
struct KvMap {
    const int32_t *pt;  // the sequence's block-table row, or nullptr (packed)
    int shift;
#ifdef SA_CHECKED
    uint32_t *check;
    __device__ __forceinline__ int row(int t) const
    {
        if (!pt)
            return t;
        int page = pt[t >> shift];
        contract_flag(check, page < 0, kCheckPage);
        page = page < 0 ? 0 : page;
        return (page << shift) | (t & ((1 << shift) - 1));
    }
#else
    __device__ __forceinline__ int row(int t) const
    {
        return pt ? (pt[t >> shift] << shift) | (t & ((1 << shift) - 1)) : t;
    }
#endif
};

__device__ __forceinline__ KvMap kv_map(const KP &P, int b)
{
    KvMap m;
    m.pt = P.block_table ? P.block_table + (long long)b * P.max_pages : nullptr;
    m.shift = P.page_shift;
#ifdef SA_CHECKED
    m.check = P.check;
#endif
    return m;
}

// A row's selection count clamped into [0, topk] (out of range: flagged by checked builds).
__device__ __forceinline__ int clamp_nsel(const KP &P, int ns)
{
    contract_flag(P.check, ns < 0 || ns > P.topk, kCheckTable);
    return ns < 0 ? 0 : (ns > P.topk ? P.topk : ns);
}

__device__ __forceinline__ long long kv_base(const KP &P, const Seq &s) { return P.block_table ? 0 : s.k_off; }

// Sequence holding packed query index i: the number of b in [1, batch) with
// cu_seqlens_q[b] <= i, counted with one load per lane and a ballot (no chain
// of dependent loads).  Every lane of the wavefront must call it with the same i.
__device__ __forceinline__ int seq_of_query(const KP &P, long long i)
{
    const int lane = threadIdx.x & (kWave - 1);
    int cnt = 0;
    for (int base = 1; base < P.batch; base += kWave) {
        int b = base + lane;
        cnt += __popcll(__ballot(b < P.batch && P.cu_q[b] <= i));
    }
    return cnt;
}

// Candidate blocks of a selection row are one contiguous range [j_lo, j_hi):
// a block is a candidate iff it ends at or before p_sel and meets the non-fixed
// region [n_init, p_sel - window + 1) (every other token up to p_sel is an init
// or window token).
__device__ __host__ __forceinline__ void cand_range(int g, int n_init, int window, int n_k, int p_sel,
                                                    int &j_lo, int &j_hi)
{
    int hi = p_sel - window + 1;
    j_lo = 0;
    j_hi = 0;
    if (p_sel < 0 || n_init >= hi)
        return;
    int nb = (n_k + g - 1) / g;
    int nb_vis = (p_sel >= n_k - 1) ? nb : (p_sel + 1) / g;
    int top = (hi + g - 1) / g;
    j_lo = n_init / g;
    j_hi = nb_vis < top ? nb_vis : top;
    if (j_hi < j_lo)
        j_hi = j_lo;
}

// Candidate range of a selection row: blocks (cand_range), or, for bucket selection,
// the buckets of the complete cluster blocks ending at or before p_sel.
__device__ __host__ __forceinline__ void row_cands(const KP &P, int n_k, int p_sel, int &j_lo, int &j_hi)
{
    if (P.bucket_nb > 0) {
        int ncb = p_sel < 0 ? 0 : (p_sel + 1) / P.bucket_c;
        ncb = ncb < n_k / P.bucket_c ? ncb : n_k / P.bucket_c;
        ncb = ncb < P.bucket_nblk ? ncb : P.bucket_nblk;
        j_lo = 0;
        j_hi = ncb * P.bucket_nb;
        return;
    }
    cand_range(P.g, P.n_init, P.window, n_k, p_sel, j_lo, j_hi);
}

// The first candidate index any row can have.
__device__ __host__ __forceinline__ int first_cand(const KP &P) { return P.bucket_nb > 0 ? 0 : P.n_init / P.g; }

// The attended set of one query as three disjoint ranges of positions:
//   [0, n1) -> init tokens; [n1, n1+n2) -> tokens of the selected blocks clipped
//   to [n_init, p_sel-window+1); [n1+n2, total) -> [lo_w, p].
struct ASet {
    int n1, n2, n3, total;
    int lo_w;
    int nsel, g;
    int start_f, len_f;   // first selected block, clipped
    int p;                // query position (tokens are clamped to <= p)
#ifdef SA_CHECKED
    uint32_t *check;
    int j_lo, j_hi;       // the row's candidate blocks: every listed block must lie in them
#endif
};

__device__ __forceinline__ ASet aset_make(const KP &P, int n_k, int p, int p_sel, const int32_t *sel, int nsel)
{
    ASet a;
    a.g = P.g;
    a.p = p < n_k - 1 ? p : n_k - 1;
    a.n1 = P.n_init < p + 1 ? P.n_init : p + 1;
    if (a.n1 < 0)
        a.n1 = 0;
    int hi = p_sel - P.window + 1;
    a.lo_w = P.n_init > hi ? P.n_init : hi;
    a.n3 = p - a.lo_w + 1;
    if (a.n3 < 0)
        a.n3 = 0;
    a.nsel = (nsel > 0 && P.n_init < hi) ? nsel : 0;
    a.n2 = 0;
    a.start_f = 0;
    a.len_f = 0;
    if (a.nsel > 0) {
        int g = P.g;
        int jf = sel[0];
        int s0 = jf * g, e0 = min((jf + 1) * g, n_k);
        a.start_f = max(s0, P.n_init);
        a.len_f = max(0, min(e0, hi) - a.start_f);
        if (a.nsel == 1) {
            a.n2 = a.len_f;
        } else {
            int jl = sel[a.nsel - 1];
            int len_l = max(0, min(min((jl + 1) * g, n_k), hi) - jl * g);
            a.n2 = a.len_f + (a.nsel - 2) * g + len_l;
        }
    }
    a.total = a.n1 + a.n2 + a.n3;
#ifdef SA_CHECKED
    a.check = P.check;
    contract_flag(P.check, p < 0 || p >= n_k, kCheckSeq);
    a.p = a.p < 0 ? 0 : a.p;
    cand_range(P.g, P.n_init, P.window, n_k, p_sel, a.j_lo, a.j_hi);
    if (a.nsel > 0)
        contract_flag(P.check, sel[0] < a.j_lo || sel[0] >= a.j_hi || sel[a.nsel - 1] < a.j_lo ||
                                   sel[a.nsel - 1] >= a.j_hi || (a.nsel > 1 && sel[a.nsel - 1] <= sel[0]),
                      kCheckTable);
#endif
    return a;
}

// Token at position pos (0 <= pos < total) of the attended set.
__device__ __forceinline__ int aset_token(const ASet &a, const int32_t *sel, int pos)
{
    int t;
    if (pos < a.n1) {
        t = pos;
    } else if (pos < a.n1 + a.n2) {
        int r = pos - a.n1;
        if (r < a.len_f) {
            t = a.start_f + r;
        } else {
            r -= a.len_f;
            int m = r / a.g;
            if (m < a.nsel - 2) {
                const int j = sel[1 + m];
#ifdef SA_CHECKED
                // a listed block inside the row's candidates, after the one before it
                contract_flag(a.check, j < a.j_lo || j >= a.j_hi || j <= sel[m], kCheckTable);
#endif
                t = j * a.g + (r - m * a.g);
            } else {
                t = sel[a.nsel - 1] * a.g + (r - (a.nsel - 2) * a.g);
            }
        }
    } else {
        t = a.lo_w + (pos - a.n1 - a.n2);
    }
#ifdef SA_CHECKED
    contract_flag(a.check, t < 0 || t > a.p, kCheckToken);
#endif
    return t < 0 ? 0 : (t > a.p ? a.p : t);   // never leave [0, p], whatever the table holds
}

// ---------------------------------------------------------------- elements

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u)             // inf / nan: keep, quiet the nan
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);                   // round to nearest, ties to even
    return (uint16_t)(u >> 16);
}

// Load 8 consecutive elements as fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8])
{
    uint4 v = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load8(const float *p, float (&x)[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t *p, const float (&x)[8])
{
    uint4 v;
    v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    v.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
    v.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = v;
}

__device__ __forceinline__ void store8(float *p, const float (&x)[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// ---------------------------------------------------------------- reductions

// v from another lane of the same 16-lane row (DPP: a VALU operand modifier, no LDS).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W lanes (W a power of two <= 64), the total in every
// lane.  Within a 16-lane row: swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), mirror each half row, mirror the row; wider groups add the
// partner row through a lane shuffle.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    if (W >= 2)
        v += dpp_f32<0xB1>(v);
    if (W >= 4)
        v += dpp_f32<0x4E>(v);
    if (W >= 8)
        v += dpp_f32<0x141>(v);
    if (W >= 16)
        v += dpp_f32<0x140>(v);
#pragma unroll
    for (int o = 16; o < W; o <<= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

// Monotone map of an fp32 score to uint32 (larger score -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (a -0 score comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(unsigned long long mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

} // namespace sa
