// attn_prefill.hip -- bf16 sparse attention on gfx950 matrix cores for many
// consecutive queries with per-query selections (prefill): queries whose
// attended sets overlap are processed together over the union of their tiles,
// each row masked to its own set (PulseCol §3.1 Eq. (2); SparDA summary,
// Method).
#include "mfma_common.hpp"

namespace sa {

// ---------------------------------------------------------------- union tiles (prefill)

// Load one 32-token key tile starting at token t0 (contiguous), with the lane's
// 8-bit live mask taken from the 32-bit token mask of its row.
template <int D>
__device__ __forceinline__ void load_tile(ChunkRegs<D> &r, int t0, int n_k, uint32_t m32, const uint16_t *kb,
                                          const uint16_t *vb, long long tstride, const KvMap &map, int rr, int g4)
{
    constexpr int KS = D / 32;
#pragma unroll
    for (int s = 0; s < 2; s++) {
        int t = min(t0 + 16 * s + rr, n_k - 1);
        long long off = (long long)map.row(t) * tstride + 8 * g4;
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
            r.v[i] = ld16(vb + (long long)map.row(t) * tstride + 8 * rr);
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
        ns = clamp_nsel(P, ns);
#ifdef SA_CHECKED
        int cj_lo, cj_hi;
        cand_range(P.g, P.n_init, P.window, s.n_k, s.q0 + qw0 + qq, cj_lo, cj_hi);
#endif
        for (int e = lane; e < ns * tpb; e += kWave) {
#ifdef SA_CHECKED
            contract_flag(P.check, sel[e / tpb] < cj_lo || sel[e / tpb] >= cj_hi, kCheckTable);
#endif
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
    const uint16_t *kb = k + (kv_base(P, s) * P.h_kv + c) * D;
    const uint16_t *vb = v + (kv_base(P, s) * P.h_kv + c) * D;
    const KvMap kmap = kv_map(P, b);
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int p = 0; p < 8; p++)
        acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    ChunkRegs<D> ra, rb;
    if (n_list > 0) {
        int t = sh_list[w][0];
        load_tile<D>(ra, t * 32, s.n_k, row_mask(t), kb, vb, tstride, kmap, rr, g4);
    }
    for (int it = 0; it < n_list; it += 2) {
        if (it + 1 < n_list) {
            int t = sh_list[w][it + 1];
            load_tile<D>(rb, t * 32, s.n_k, row_mask(t), kb, vb, tstride, kmap, rr, g4);
        }
        compute_chunk<D>(ra, ra.live, qop, P.scale_log2, g4, m_run, l_part, acc);
        if (it + 1 >= n_list)
            break;
        if (it + 2 < n_list) {
            int t = sh_list[w][it + 2];
            load_tile<D>(ra, t * 32, s.n_k, row_mask(t), kb, vb, tstride, kmap, rr, g4);
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

// The wavefronts of a workgroup share each 64-token K/V tile through LDS.  A
// workgroup owns 256/G consecutive queries (64 for G = 4), 16 row tiles of 16 rows
// (G heads of 16/G queries each), spread over its wavefronts.  The workgroup's tile list is the union
// of its queries' init tiles, windows and selected blocks (block = tile, g = 64);
// for each listed tile a 64-bit mask says which of its queries selected it.  The
// list is walked in lockstep, kWgStep tiles per barrier: while step i's tiles are
// computed from one LDS buffer, step i+1's tiles are written from registers into
// the other and step i+2's loads are in flight.  Fewer barriers let the
// wavefronts' uneven per-tile work (a wavefront skips the MFMA work of tiles none
// of its rows attends) even out within a step.
constexpr int kWgMaxTiles = 2048;              // 64-token tiles per sequence (max_k <= 131072)
constexpr int kWgStep = 2;                     // tiles per barrier step (per LDS buffer)
constexpr int kWgPitch = 272;                  // LDS bytes per staged 256-byte row (bank spread)

// A thread's share of one staged 32 KB K/V tile: 2048 pieces of 16 B over NT threads.
template <int NT>
struct WgStage {
    u32x4 c[2048 / NT];
};

template <int NT>
__device__ __forceinline__ void wg_issue(WgStage<NT> &st, const uint16_t *kb, const uint16_t *vb, long long tstride,
                                         const KvMap &map, int t0, int n_k, int tid)
{
    // 2048 chunks: 128 rows (64 K, 64 V) x 16; chunk c + 1024 is the V piece of K
    // piece c (same token, same column), so each token offset serves both
    constexpr int UH = 1024 / NT;
#pragma unroll
    for (int u = 0; u < UH; u++) {
        const int chunk = tid + NT * u;
        const int row = chunk >> 4, col = chunk & 15;
        const int t = min(max(t0 + row, 0), n_k - 1);
        // row and stride are non-negative 32-bit values: one 32 x 32 -> 64-bit product
        const unsigned long long off =
            (unsigned long long)(unsigned)map.row(t) * (unsigned)tstride + (unsigned)(8 * col);
        st.c[u] = ld16(kb + off);
        st.c[u + UH] = ld16(vb + off);
    }
}

template <int NT>
__device__ __forceinline__ void wg_write(const WgStage<NT> &st, unsigned char *buf, int tid)
{
#pragma unroll
    for (int u = 0; u < 2048 / NT; u++) {
        const int chunk = tid + NT * u;
        const int row = chunk >> 4, col = chunk & 15;
        *reinterpret_cast<u32x4 *>(buf + row * kWgPitch + 16 * col) = st.c[u];
    }
}

// S^T = K Q^T of one 32-token half of a staged tile for the wavefront's MT row
// tiles (K operands read from LDS once, used by each).
template <int MT>
__device__ __forceinline__ void wg_qk(const unsigned char *buf, int h, int rr, int g4, const bf16x8 (&qop)[MT][4],
                                      f32x4 (&st)[MT][2])
{
#pragma unroll
    for (int a = 0; a < MT; a++)
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
        for (int a = 0; a < MT; a++)
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
template <int MT>
__device__ __forceinline__ void wg_pv(const unsigned char *buf, int h, int rr, int g4, const bf16x8 (&aop)[MT],
                                      f32x4 (&acc)[MT][9])
{
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int a = 0; a < MT; a++)
        acc[a][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[a], ones, acc[a][8], 0, 0, 0);
    const unsigned char *vr = buf + (64 + 32 * h + 4 * g4 + (rr >> 2)) * kWgPitch + 8 * (rr & 3);
#pragma unroll
    for (int p = 0; p < 8; p++) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vr + 32 * p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vr + 16 * kWgPitch + 32 * p));
        const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int a = 0; a < MT; a++)
            acc[a][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[a], bop, acc[a][p], 0, 0, 0);
    }
}

// One staged 64-token tile for the wavefront's two 16-row tiles (this lane: row
// rr of each, 8 logits per 32-token half).  Both QK products come first; the
// reference max m_run is kept on raw logits (the scale is positive) and moves
// lazily, at most once per tile: only when the tile's max exceeds it by more than
// `lazy` (2^8 after scaling), so unnormalised weights stay below 256 and the
// output accumulators are rescaled rarely (a wavefront-uniform branch).  Any
// reference gives the same normalised result (the offset -m_run * scale is kept
// with it, so the common path only compares).  A lane whose 8 logits of a half
// are all masked gets offset -inf there, so its weights are exp2(-inf) = 0
// without a select per logit; per-logit masks (a -1e30 sentinel,
// which underflows to 0) are applied only when some lane has a partly live half
// (causal edge, window or sink boundary).  exp2 is the hardware instruction
// (results below 2^-126 flush to zero, which the sum cannot see next to the
// reference term).  Row sums come from the P V product itself (a ones column
// tile), so the accumulators carry them and their rescaling.
// Maxima of matrix-core results as single instructions: fmaxf first quiets both
// operands of a two-way maximum (two more instructions each), which a logit that
// is never a signalling NaN does not need.
__device__ __forceinline__ float max2(float a, float b)
{
    float r;
    __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float max3(float a, float b, float c)
{
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Maximum with lane i ^ 16 / lane i ^ 32 (gfx950 lane swaps between 16-lane rows /
// 32-lane halves, no LDS permute): each lane ends up with its own value in one
// result and its partner's in the other.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int MT>
__device__ __forceinline__ void wg_tile(const unsigned char *buf, int rr, int g4, const bf16x8 (&qop)[MT][4],
                                        const uint32_t (&live)[2][MT], bool partial, float scale_log2, float lazy,
                                        float (&m_run)[MT], float (&neg)[MT], f32x4 (&acc)[MT][9])
{
    f32x4 st[2][MT][2];                                   // [half][row tile][16-token subtile]
    wg_qk<MT>(buf, 0, rr, g4, qop, st[0]);
    wg_qk<MT>(buf, 1, rr, g4, qop, st[1]);
    if (partial) {                       // finite sentinel: far below any live logit
        // keep this a branch: executed unconditionally (as selects) it costs ~100
        // vector instructions per tile, and it is needed only at set boundaries
        __asm__ volatile("" ::);
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int a = 0; a < MT; a++)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    st[h][a][i >> 2][i & 3] = (live[h][a] >> i) & 1u ? st[h][a][i >> 2][i & 3] : -1e30f;
    }
    float mcs[MT];
    bool bump[MT];
#pragma unroll
    for (int a = 0; a < MT; a++) {
        float mhv[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {                     // chained three-way maxima
            const f32x4 *x = st[h][a];
            float mh = max3(x[0][0], x[0][1], x[0][2]);
            mh = max3(mh, x[0][3], x[1][0]);
            mh = max3(mh, x[1][1], x[1][2]);
            mh = max2(mh, x[1][3]);
            mhv[h] = live[h][a] != 0u ? mh : -INFINITY;
        }
        float mc = max2(mhv[0], mhv[1]);
        mc = max_xor16(mc);
        mc = max_xor32(mc);
        mcs[a] = mc;
        bump[a] = mc > m_run[a] + lazy;
    }
    bool any_bump = false;
#pragma unroll
    for (int a = 0; a < MT; a++)
        any_bump = any_bump || bump[a];
    if (__ballot(any_bump)) {
        // the reference moves (rarely): the offset -m_run * scale and the accumulators follow
#pragma unroll
        for (int a = 0; a < MT; a++) {
            const float m_old = m_run[a];
            m_run[a] = bump[a] ? mcs[a] : m_run[a];
            neg[a] = bump[a] ? -m_run[a] * scale_log2 : neg[a];
            const float alpha = bump[a] ? __builtin_amdgcn_exp2f(fmaf(m_old, scale_log2, neg[a])) : 1.f;
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
        bf16x8 aop[MT];
#pragma unroll
        for (int a = 0; a < MT; a++) {
            // a dead half gets offset -inf: its (finite) logits weigh exp2(-inf) = 0
            const float n_eff = live[h][a] != 0u ? neg[a] : -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; i++)
                aop[a][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(st[h][a][i >> 2][i & 3], scale_log2, n_eff));
        }
        wg_pv<MT>(buf, h, rr, g4, aop, acc);
    }
}

// The 8 logits of lane group g4 are tokens 4*g4 .. +3 and 16 + 4*g4 .. +3 of the chunk.
__device__ __forceinline__ uint32_t live8(uint32_t m32, int g4)
{
    return ((m32 >> (4 * g4)) & 0xfu) | (((m32 >> (16 + 4 * g4)) & 0xfu) << 4);
}


// NW wavefronts of MT 16-row tiles each (NW * MT = 16: 256 rows, 64 queries at G = 4).
// MT = 2 reads each staged K/V operand once for two row tiles (half the LDS traffic per
// MFMA); MT = 1 halves the registers, so twice the wavefronts share each SIMD.
template <int NW, int MT>
__global__ __launch_bounds__(64 * NW, 1) void attn_wg_kernel(KP P, const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v,
                                                             const int32_t *__restrict__ idx,
                                                             const int32_t *__restrict__ n_idx,
                                                             uint16_t *__restrict__ out, float *__restrict__ lse,
                                                             int n_qtile)
{
    constexpr int D = 128, KS = D / 32, NT = 64 * NW;
    static_assert(NW * MT == 16, "a workgroup holds 16 row tiles");
    // per tile: queries that selected it; after the list is built, entry i is the mask
    // of list entry i
    __shared__ unsigned long long sh_qm[kWgMaxTiles];
    __shared__ unsigned short sh_list[kWgMaxTiles];
    __shared__ __attribute__((aligned(16))) unsigned char sh_kv[2][kWgStep * 128 * kWgPitch];
    __shared__ int sh_scan[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its spans and tests stay scalar
    const int rr = lane & 15, g4 = lane >> 4;
    // Workgroups in launch order: each (sequence, KV head) in turn, its query tiles
    // from the last (the longest sets) to the first, so the short ones fill the tail
    // (23.5 against 23.8 ms at 128K for XCD-contiguous ranges in ascending order).
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    const long long item = blockIdx.x;
    if (item >= n_items)
        return;
    const int qt = n_qtile - 1 - (int)(item % n_qtile);
    const int c = (int)((item / n_qtile) % P.h_kv);
    const int b = (int)(item / ((long long)n_qtile * P.h_kv));
    const Seq s = seq_info(P, b);
    const int QPW = 16 * MT / P.G;                        // queries per wavefront
    const int qwg = NW * QPW;                             // queries per workgroup (<= 64)
    const int q_lo = qt * qwg;
    const int nq = max(0, min(qwg, s.n_q - q_lo));
    if (nq == 0)                                          // query tile past this sequence's queries
        return;
    const int ntile = (s.n_k + 63) / 64;

    for (int x = tid; x < ntile; x += NT)
        sh_qm[x] = 0ull;
    __syncthreads();
    for (int x = tid; x < nq * P.topk; x += NT) {
        const int qq = x / P.topk, e = x % P.topk;
        const long long qi = s.q_off + q_lo + qq;
        int ns = n_idx[(long long)c * P.rows + qi];
        ns = clamp_nsel(P, ns);
        if (e < ns) {
            const int j = idx[((long long)c * P.rows + qi) * P.topk + e];
#ifdef SA_CHECKED
            int cj_lo, cj_hi;
            cand_range(P.g, P.n_init, P.window, s.n_k, s.q0 + q_lo + qq, cj_lo, cj_hi);
            contract_flag(P.check, j < cj_lo || j >= cj_hi, kCheckTable);
#endif
            if (j >= 0 && j < ntile)
                atomicOr(&sh_qm[j], 1ull << qq);
        }
    }
    __syncthreads();
    // union list: selected blocks, init tiles, window tiles of the workgroup's queries
    const int p_first = s.q0 + q_lo, p_last = s.q0 + q_lo + nq - 1;
    const int init_hi = (min(P.n_init, p_last + 1) + 63) / 64;
    const int win_lo = max(P.n_init, p_first - P.window + 1) / 64, win_hi = p_last / 64;
    constexpr int kPer = kWgMaxTiles / NT;                // tiles per thread
    const int per = (ntile + NT - 1) / NT;
    unsigned long long qv[kPer];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; u++) {
        const int j = tid * per + u;
        qv[u] = u < per && j < ntile ? sh_qm[j] : 0ull;
        cnt += (u < per && j < ntile && (qv[u] != 0ull || j < init_hi || (j >= win_lo && j <= win_hi))) ? 1 : 0;
    }
    int2 sc = block_scan_int_nt<NT>(cnt, sh_scan);       // ends with a barrier: every read is done
    int pos = sc.x;
#pragma unroll
    for (int u = 0; u < kPer; u++) {
        const int j = tid * per + u;
        if (u < per && j < ntile && (qv[u] != 0ull || j < init_hi || (j >= win_lo && j <= win_hi))) {
            sh_list[pos] = (unsigned short)j;
            sh_qm[pos] = qv[u];                          // compacted in place
            pos++;
        }
    }
    const int n_list = sc.y;
    __syncthreads();                                      // the list is complete

    // this wavefront's rows: a = 0 .. MT-1 -> rows 16a + rr of its 16 MT
    const long long tstride = (long long)P.h_kv * D;
    const uint16_t *kb = k + (kv_base(P, s) * P.h_kv + c) * D;
    const uint16_t *vb = v + (kv_base(P, s) * P.h_kv + c) * D;
    const KvMap kmap = kv_map(P, b);
    bf16x8 qop[MT][KS];
    int p_row[MT], lo_w[MT], qbit[MT];
    bool row_ok[MT];
#pragma unroll
    for (int a = 0; a < MT; a++) {
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
    // the wave's rows' window starts span [w_lo_min, w_lo_max]
    const int w_lo_min = max(P.n_init, wp_first - P.window + 1), w_lo_max = max(P.n_init, wp_last - P.window + 1);

    float m_run[MT], neg_run[MT];                         // reference max (raw logits), -m_run * scale
    const float lazy = 8.f / P.scale_log2;
    f32x4 acc[MT][9];                                     // [8]: row sums (ones column tile)
#pragma unroll
    for (int a = 0; a < MT; a++) {
        m_run[a] = -INFINITY;
        neg_run[a] = 0.f;                                 // set with m_run at a row's first live tile
#pragma unroll
        for (int p = 0; p < 9; p++)
            acc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One listed tile e from a staged buffer: this wavefront's rows that attend it (its
    // masks per 32-token half and row tile), then the tile's MFMA work if any row is live.
    auto compute_tile = [&](int e, const unsigned char *buf) {
        const int tile = sh_list[e];
        const unsigned long long qm = sh_qm[e];
        uint32_t live[2][MT];
        bool any = false, part = false;
        const int t_lo = tile * 64, t_hi = t_lo + 63;
        if ((t_lo >= P.n_init && t_hi < w_lo_min) || ((t_lo >= w_lo_max || t_hi < P.n_init) && t_hi <= wp_first)) {
            // tile wholly before every row's window and past the sinks (live where
            // selected), or wholly inside every row's window or sinks
            const bool fixed = t_lo < P.n_init || t_lo >= w_lo_max;
#pragma unroll
            for (int a = 0; a < MT; a++) {
                const bool on = row_ok[a] && (fixed || ((qm >> qbit[a]) & 1ull));
                live[0][a] = live[1][a] = on ? 0xffu : 0u;
                any = any || on;
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int t0 = t_lo + 32 * h;
#pragma unroll
                for (int a = 0; a < MT; a++) {
                    const bool sb = (qm >> qbit[a]) & 1ull;
                    live[h][a] = row_ok[a] ? live8(tile_mask(t0, p_row[a], P.n_init, lo_w[a], sb), g4) : 0u;
                    any = any || live[h][a] != 0u;
                    part = part || (live[h][a] != 0u && live[h][a] != 0xffu);
                }
            }
        }
        if (__ballot(any) != 0ull)
            wg_tile<MT>(buf, rr, g4, qop, live, __ballot(part) != 0ull, P.scale_log2, lazy, m_run, neg_run, acc);
    };
    // whether this wavefront's rows can attend listed tile e at all
    auto needs = [&](int e) {
        const int tile = sh_list[e];
        return (sh_qm[e] & wmask) != 0ull || tile < w_init_hi || (tile >= w_win_lo && tile <= w_win_hi);
    };

    // Every query attends at least its own position (window >= 1), so n_list >= 1
    // here; the staging below reads sh_list[0 .. n_list) only.  Load issues are
    // unconditional (clamped to the last tile) so the load counters the compiler
    // tracks are the same on every path.
    WgStage<NT> stage[kWgStep];
    const int last = max(n_list - 1, 0);
    constexpr int kTileBytes = 128 * kWgPitch;
    if (n_list > 0) {
        // Step i: barrier (LDS buffer i&1 holds tiles kWgStep*i ..), compute those
        // tiles, write step i+1's tiles from registers into the other buffer, then
        // issue the loads of step i+2.
#pragma unroll
        for (int x = 0; x < kWgStep; x++)
            wg_issue<NT>(stage[x], kb, vb, tstride, kmap, sh_list[min(x, last)] * 64, s.n_k, tid);
#pragma unroll
        for (int x = 0; x < kWgStep; x++) {
            wg_write<NT>(stage[x], sh_kv[0] + x * kTileBytes, tid);
            wg_issue<NT>(stage[x], kb, vb, tstride, kmap, sh_list[min(kWgStep + x, last)] * 64, s.n_k, tid);
        }
        const int n_step = (n_list + kWgStep - 1) / kWgStep;
        for (int i = 0; i < n_step; i++) {
            __syncthreads();                                   // LDS buffer i&1 holds step i's tiles
#pragma unroll
            for (int x = 0; x < kWgStep; x++) {
                const int e = kWgStep * i + x;
                if (e < n_list && needs(e))
                    compute_tile(e, sh_kv[i & 1] + x * kTileBytes);
            }
#pragma unroll
            for (int x = 0; x < kWgStep; x++) {
                wg_write<NT>(stage[x], sh_kv[(i + 1) & 1] + x * kTileBytes, tid);
                wg_issue<NT>(stage[x], kb, vb, tstride, kmap, sh_list[min(kWgStep * (i + 2) + x, last)] * 64, s.n_k,
                             tid);
            }
        }
    }
    // Epilogue: lane (rr, g4) holds d = 16 p + rr of rows 4 g4 + r4; normalised bf16
    // rows are transposed through this wavefront's 16 MT-row slice of the (now
    // idle) staging buffers and stored as 16-byte row pieces.
    __syncthreads();
    unsigned char *ob = &sh_kv[0][0] + w * 16 * MT * kWgPitch;
#pragma unroll
    for (int a = 0; a < MT; a++) {
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
    for (int t = 0; t < 4 * MT; t++) {
        const int u = lane + 64 * t;                       // 256 MT pieces: 16 MT rows x 16
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
    // 8 wavefronts of two row tiles: 16 wavefronts of one (four per SIMD, twice the LDS
    // operand traffic per MFMA) measured 21.7 against 21.4 ms at 128K
    constexpr int NW = 8, MT = 2;
    const int qwg = NW * (16 * MT / P.G);
    const int n_qtile = (P.max_q + qwg - 1) / qwg;
    const long long n_items = (long long)n_qtile * P.batch * P.h_kv;
    if (ev0 && ev1)
        (void)hipEventRecord((hipEvent_t)ev0, st);
    attn_wg_kernel<NW, MT><<<dim3((unsigned)n_items), dim3(64 * NW), 0, st>>>(
        P, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, idx, n_idx, (uint16_t *)out, lse, n_qtile);
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

} // namespace sa
