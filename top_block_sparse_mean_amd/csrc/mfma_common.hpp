// mfma_common.hpp -- operand layouts and the 32-token chunk step shared by the
// bf16 matrix-core attention kernels (decode gather and prefill union tiles).
// Online softmax with fp32 running max / sum / output (PulseCol §3.1 Eq. (2);
// S3R review, sparse drafting formula).
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
#pragma once
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

// Loads the K and V rows of list entries base .. base+31 (tok[] holds each entry's
// row relative to kb / vb).  An entry is live for the lane's row when it lies in
// the split (pos < n) and below the row's causal limit lim: the attended list is
// ascending in position, so a row that stops d positions before the unit's last
// query drops exactly the list's last d entries.
template <int D>
__device__ __forceinline__ void load_chunk(ChunkRegs<D> &r, const int *tok, int base, int n, const uint16_t *kb,
                                           const uint16_t *vb, long long tstride, int rr, int g4, int lim)
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
        r.live |= (pos < n && pos < lim) ? (1u << i) : 0u;
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
// Splits of one attended set: attn_combine reads one split per lane of a wavefront.
constexpr int kMaxSplits = 64;

// Exclusive scan of one int per thread over an NT-thread workgroup; (exclusive, total).
// sh holds NT / 64 ints.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ int2 block_scan_int_nt(int v, int *sh)
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
    for (int i = 0; i < NT / kWave; i++) {
        int c = sh[i];
        off += i < w ? c : 0;
        tot += c;
    }
    __syncthreads();
    return make_int2(off + incl - v, tot);
}
constexpr int kSelCap = 4096;

} // namespace sa
