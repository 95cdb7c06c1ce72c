// bucket.hip -- the LSA flat bucket index (LSA deep-read, §2.2-§2.3).
//
// Build: the pooled keys of every complete cluster block (C consecutive tokens =
// M = C/g pooled groups of one sequence and KV head) are clustered bottom-up by
// Ward's criterion.  Every round, each bucket finds its cheapest partner among the
// buckets it may join (merged size <= cap/g groups); pairs that are each other's
// cheapest merge together -- only the cheapest (by cost, then name) when all of
// them would leave fewer than NB buckets.  A bucket is named by its smallest
// member.  Ward's cost of buckets A, B (member sums S, sizes n) is
// |n_B S_A - n_A S_B|^2 / (n_A n_B (n_A + n_B)), accumulated with fused
// multiply-adds over the head dimension in order, lower name first.  The result
// per block: members grouped by bucket (buckets in name order, members ascending),
// NB + 1 offsets, and NB centroids (normalised member sums).  One workgroup per
// block keeps the sums (M x d) and the pair costs (M x M) in LDS.
//
// Select: the group's summed selector query scores the centroids of the complete
// blocks that end at or before the row's selection position (the ordinary
// scoring and top-k kernels, run over the centroid table), and the chosen buckets
// are expanded to their member groups, sorted ascending into the row's table.
#include "mfma_common.hpp"
#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

constexpr int kBucketMaxM = 128;     // pooled groups per cluster block

__device__ __forceinline__ float ward_cost(const float *sa, int na, const float *sb, int nb, int d)
{
    float acc = 0.0f;
    const float fa = (float)na, fb = (float)nb;
    for (int e = 0; e < d; e++) {
        const float t = fa * sb[e];
        const float diff = fmaf(fb, sa[e], -t);
        acc = fmaf(diff, diff, acc);
    }
    return acc * (1.0f / (float)(na * nb * (na + nb)));
}

// grid: h_kv * batch * nblk workgroups of NT threads, one per (KV head, sequence, block).
// The sums and costs take most of a CU's LDS, so one workgroup runs per CU: NT = 1024
// puts four wavefronts on each SIMD to cover the LDS latency of the cost loops (with one
// wavefront per SIMD a round took about 125 us).  Member sums are kept at a pitch of
// D + 1 floats, so the lanes of a wavefront, each on its own partner bucket, read
// distinct LDS banks at every step of the cost loop.
template <int D, int NT>
__global__ __launch_bounds__(NT) void bucket_build_kernel(KP P, const float *__restrict__ k_cmp, BucketArgs B)
{
    constexpr int PS = D + 1;
    __shared__ float sh_s[kBucketMaxM * PS];
    __shared__ float sh_w[kBucketMaxM * kBucketMaxM];
    __shared__ int sh_size[kBucketMaxM], sh_alive[kBucketMaxM], sh_root[kBucketMaxM], sh_nn[kBucketMaxM];
    __shared__ int sh_into[kBucketMaxM], sh_pair[kBucketMaxM], sh_bk[kBucketMaxM], sh_off[kBucketMaxM + 1];
    __shared__ float sh_nnc[kBucketMaxM];
    __shared__ int sh_chg[kBucketMaxM];       // merged or absorbed in the last round: its costs change
    const int M = B.C / P.g, capg = B.cap / P.g, NB = B.NB;
    const int span = B.nblk - B.from;                            // blocks from B.from on
    const int blk = B.from + (int)(blockIdx.x % span);
    const int b = (int)((blockIdx.x / span) % P.batch);
    const int c = (int)(blockIdx.x / ((long long)span * P.batch));
    const long long item = ((long long)c * P.batch + b) * B.nblk + blk;
    const int tid = threadIdx.x;
    const Seq s = seq_info(P, b);
    int32_t *mem = B.member + item * M;
    int32_t *off = B.offset + item * (NB + 1);
    float *cen = B.centroid + item * (long long)NB * D;
    if ((long long)(blk + 1) * B.C > s.n_k) {                 // incomplete block: no buckets
        for (int x = tid; x < M; x += NT)
            mem[x] = -1;
        for (int x = tid; x <= NB; x += NT)
            off[x] = 0;
        return;
    }
    const float *src = k_cmp + (((long long)c * P.batch + b) * P.nb_max + (long long)blk * M) * D;
    for (int x = tid; x < M * D; x += NT)
        sh_s[(x / D) * PS + x % D] = src[x];
    for (int x = tid; x < M; x += NT) {
        sh_size[x] = 1;
        sh_alive[x] = 1;
        sh_root[x] = x;
        sh_chg[x] = 1;
    }
    int count = M;
    // the per-bucket searches of a round: LP consecutive lanes per bucket
    constexpr int LP = NT / kBucketMaxM;
    static_assert(LP >= 1 && LP <= kWave && (LP & (LP - 1)) == 0, "lanes per bucket: a power of two within a wavefront");
    const int r_lp = tid / LP, part_lp = tid % LP;
    __syncthreads();
    while (count > NB) {
        // pair costs, lower name first; a pair of two unchanged buckets keeps its cost
        // (the same arithmetic on the same sums and sizes)
        for (int pi = tid; pi < M * M; pi += NT) {
            const int a = pi / M, o = pi % M;
            if (o <= a || !(sh_chg[a] | sh_chg[o]))
                continue;
            float wv = INFINITY;
            if (sh_alive[a] && sh_alive[o] && sh_size[a] + sh_size[o] <= capg)
                wv = ward_cost(sh_s + a * PS, sh_size[a], sh_s + o * PS, sh_size[o], D);
            sh_w[a * M + o] = wv;
            sh_w[o * M + a] = wv;
        }
        __syncthreads();
        {   // cheapest partner, ties to the lower name: the (cost, name) minimum of a bucket's
            // row, LP lanes each over the partners o = part (mod LP), then combined
            int best = -1;
            float bc = INFINITY;
            if (r_lp < M && part_lp < M && sh_alive[r_lp]) {
                const int n8 = (M - part_lp + LP - 1) / LP;   // partners of this lane (>= 1)
                const int rot = r_lp % n8;                    // rotated start: the rows hit distinct banks
                for (int i = 0; i < n8; i++) {
                    const int o = part_lp + LP * (i + rot < n8 ? i + rot : i + rot - n8);
                    const float wv = o == r_lp ? INFINITY : sh_w[r_lp * M + o];
                    if (wv < bc || (wv == bc && wv < INFINITY && o < best)) {
                        bc = wv;
                        best = o;
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < LP; off <<= 1) {
                const float oc = __shfl_xor(bc, off, kWave);
                const int ob = __shfl_xor(best, off, kWave);
                if (ob >= 0 && (oc < bc || (oc == bc && (best < 0 || ob < best)))) {
                    bc = oc;
                    best = ob;
                }
            }
            if (r_lp < M && part_lp == 0) {
                sh_nn[r_lp] = best;
                sh_nnc[r_lp] = bc;
                sh_into[r_lp] = -1;
            }
        }
        __syncthreads();
        bool pr = false;
        if (tid < M) {
            const int o = sh_nn[tid];
            pr = sh_alive[tid] && o > tid && sh_nn[o] == tid;
            sh_pair[tid] = pr ? 1 : 0;
        }
        const int np = __syncthreads_count(pr);
        const int take = np < count - NB ? np : count - NB;
        if (take == 0)
            break;
        {   // rank by (cost, name) among the pairs: LP lanes per pair, each over every LP-th bucket
            const bool rp = r_lp < M && sh_pair[r_lp];
            int rank = 0;
            if (rp) {
                const float cr = sh_nnc[r_lp];
                for (int a = part_lp; a < M; a += LP)
                    if (sh_pair[a] && (sh_nnc[a] < cr || (sh_nnc[a] == cr && a < r_lp)))
                        rank++;
            }
#pragma unroll
            for (int off = 1; off < LP; off <<= 1)
                rank += __shfl_xor(rank, off, kWave);
            if (rp && part_lp == 0 && rank < take)
                sh_into[sh_nn[r_lp]] = r_lp;
        }
        __syncthreads();
        for (int x = tid; x < M * D; x += NT) {             // S_a += S_o (pairs are disjoint)
            const int a = sh_into[x / D];
            if (a >= 0)
                sh_s[a * PS + x % D] += sh_s[(x / D) * PS + x % D];
        }
        if (tid < M)
            sh_chg[tid] = 0;
        __syncthreads();
        if (tid < M && sh_into[tid] >= 0) {
            atomicAdd(&sh_size[sh_into[tid]], sh_size[tid]);
            sh_alive[tid] = 0;
            sh_chg[tid] = 1;
            sh_chg[sh_into[tid]] = 1;
        }
        __syncthreads();
        if (tid < M) {
            const int r = sh_root[tid];
            if (sh_into[r] >= 0)
                sh_root[tid] = sh_into[r];
        }
        count -= take;
        __syncthreads();
    }
    // buckets in name order: index, offsets, members ascending within each bucket
    if (tid < M) {
        int k = 0, o = 0;
        for (int a = 0; a < tid; a++)
            if (sh_alive[a]) {
                k++;
                o += sh_size[a];
            }
        sh_bk[tid] = k;
        if (sh_alive[tid] && k < NB)
            sh_off[k] = o;
    }
    __syncthreads();
    if (tid < M) {
        const int r = sh_root[tid], k = sh_bk[r];
        int pos = 0;
        for (int y = 0; y < tid; y++)
            pos += sh_root[y] == r ? 1 : 0;
        if (k < NB)
            mem[sh_off[k] + pos] = tid;
    }
    if (tid < NB)
        off[tid] = sh_off[tid];
    if (tid == 0)
        off[NB] = M;
    // centroids: one wavefront per bucket
    const int w = tid / kWave, lane = tid % kWave;
    for (int a = w; a < M; a += NT / kWave) {
        if (!sh_alive[a] || sh_bk[a] >= NB)
            continue;
        float ss = 0.f;
        for (int e = lane; e < D; e += kWave)
            ss += sh_s[a * PS + e] * sh_s[a * PS + e];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            ss += __shfl_xor(ss, o, kWave);
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        for (int e = lane; e < D; e += kWave)
            cen[(long long)sh_bk[a] * D + e] = sh_s[a * PS + e] * inv;
    }
}

// grid: (rows, h_kv), 256 threads.  The row's chosen buckets (ascending) are expanded
// to their member groups (block * M + member); groups wholly inside the sink or the
// window are left out (they are attended anyway, as for block candidates), so the
// table keeps the attention's shape: only its first group may reach into the sink
// and only its last into the window.  Written ascending, -1 padded to the row's table
// of width P.topk.  The chosen buckets ascend by block, so the groups of different
// blocks are already in order and only a block's own buckets interleave: each block
// of the row (a segment) marks its kept members in a 128-bit mask, and the segments
// emit their set bits in order at offsets from a scan of their counts.  A group
// belongs to one bucket, so the list has no repeats.  The host keeps the expansion
// within the table (topk >= n_buckets * cap / g, topk <= 4096).
__global__ __launch_bounds__(256) void bucket_expand_kernel(KP P, BucketArgs B, const int32_t *__restrict__ tbl,
                                                            const int32_t *__restrict__ tn, int kb,
                                                            int32_t *__restrict__ idx, int32_t *__restrict__ n_idx)
{
    constexpr int NT = 256, PER = 4;                      // chosen buckets per thread (kb <= 1024)
    constexpr int MW = kBucketMaxM / 32;                  // mask words per segment
    __shared__ uint32_t sh_mask[NT * PER * MW];
    __shared__ int sh_segblk[NT * PER];
    __shared__ int sh_scan[NT / kWave];
    const long long row = blockIdx.x;
    const int c = blockIdx.y, tid = threadIdx.x;
    const int M = B.C / P.g, NB = B.NB;
    const int b = P.shared ? (int)row : seq_of_query(P, row);
    const Seq sq = seq_info(P, b);
    const int p_sel = P.shared ? sq.q0 - 1 : sq.q0 + (int)(row - sq.q_off);
    const int hi = p_sel - P.window + 1;                 // the window starts here
    const long long base_bc = ((long long)c * P.batch + b) * B.nblk;
    int nsel = tn[(long long)c * P.rows + row];
    nsel = nsel < 0 ? 0 : (nsel > kb ? kb : nsel);
    const int32_t *t = tbl + ((long long)c * P.rows + row) * kb;
    // this thread's chosen buckets and whether each starts a new block (segment)
    int blk_of[PER], lb_of[PER];
    bool starts[PER];
    int nstart = 0;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int sidx = tid * PER + u;
        blk_of[u] = -1;
        lb_of[u] = 0;
        starts[u] = false;
        if (sidx < nsel) {
            const int j = t[sidx];
            blk_of[u] = j / NB;
            lb_of[u] = j % NB;
            starts[u] = sidx == 0 || t[sidx - 1] / NB != blk_of[u];
            nstart += starts[u] ? 1 : 0;
        }
    }
    const int2 ss = block_scan_int_nt<NT>(nstart, sh_scan);   // ends with a barrier
    const int nseg = ss.y;
    for (int x = tid; x < nseg * MW; x += NT)
        sh_mask[x] = 0u;
    int seg = ss.x - 1;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        seg += starts[u] ? 1 : 0;
        if (starts[u])
            sh_segblk[seg] = blk_of[u];
    }
    __syncthreads();
    // each kept member sets its bit in its block's mask
    seg = ss.x - 1;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        seg += starts[u] ? 1 : 0;
        if (blk_of[u] < 0)
            continue;
        const int32_t *off = B.offset + (base_bc + blk_of[u]) * (NB + 1);
        const int32_t *mem = B.member + (base_bc + blk_of[u]) * M;
        for (int x = off[lb_of[u]]; x < off[lb_of[u] + 1]; x++) {
            const int m = mem[x], grp = blk_of[u] * M + m;
            if (grp * P.g < hi && (grp + 1) * P.g > P.n_init)
                atomicOr(&sh_mask[seg * MW + (m >> 5)], 1u << (m & 31));
        }
    }
    __syncthreads();
    // segments in order: counts, a scan, then each segment's groups ascending
    int cnt[PER], mine = 0;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int sg = tid * PER + u;
        cnt[u] = 0;
        if (sg < nseg)
#pragma unroll
            for (int q = 0; q < MW; q++)
                cnt[u] += __popc(sh_mask[sg * MW + q]);
        mine += cnt[u];
    }
    const int2 os = block_scan_int_nt<NT>(mine, sh_scan);
    const int kept = os.y;
    int32_t *out = idx + ((long long)c * P.rows + row) * P.topk;
    int pos = os.x;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int sg = tid * PER + u;
        if (sg >= nseg)
            continue;
        const int gb = sh_segblk[sg] * M;
#pragma unroll
        for (int q = 0; q < MW; q++) {
            uint32_t bits = sh_mask[sg * MW + q];
            while (bits) {
                const int bit = __ffs(bits) - 1;
                bits &= bits - 1;
                if (pos < P.topk)
                    out[pos] = gb + 32 * q + bit;
                pos++;
            }
        }
    }
    for (int x = kept + tid; x < P.topk; x += NT)
        out[x] = -1;
    if (tid == 0)
        n_idx[(long long)c * P.rows + row] = kept;
}

hipError_t launch_bucket_build(const KP &P, const float *k_cmp, const BucketArgs &B, hipStream_t st)
{
    if (B.from >= B.nblk)
        return hipSuccess;
    const long long items = (long long)P.h_kv * P.batch * (B.nblk - B.from);
    constexpr int NT = 1024;
    if (P.d == 128)
        bucket_build_kernel<128, NT><<<dim3((unsigned)items), dim3(NT), 0, st>>>(P, k_cmp, B);
    else
        bucket_build_kernel<64, NT><<<dim3((unsigned)items), dim3(NT), 0, st>>>(P, k_cmp, B);
    return hipGetLastError();
}

// The selection's parameters for the centroid table: candidates are buckets, the
// table rows are centroids (pooled-row addressing), k is the bucket count.
KP bucket_select_kp(const KP &P, const BucketArgs &B, int kb)
{
    KP q = P;
    q.bucket_c = B.C;
    q.bucket_nb = B.NB;
    q.bucket_nblk = B.nblk;
    q.nb_max = B.nblk * B.NB;
    q.g = P.g > 1 ? P.g : 2;         // any g > 1: centroid rows are addressed like pooled keys
    q.topk = kb;
    q.topk_per_seq = nullptr;
    q.select_mode = 0;
    q.pool_overlap = 0;
    return q;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t bucket_select_workspace_bytes(const KP &P, const BucketArgs &B, int kb)
{
    const KP q = bucket_select_kp(P, B, kb);
    return align256(select_workspace_bytes(q, select_plan(q))) +
           align256((size_t)P.h_kv * (size_t)P.rows * (size_t)kb * sizeof(int32_t)) +
           align256((size_t)P.h_kv * (size_t)P.rows * sizeof(int32_t));
}

hipError_t launch_bucket_select(const KP &P, int dtype, const void *q_sel, const BucketArgs &B, int kb, int32_t *idx,
                                int32_t *n_idx, void *ws, hipStream_t st)
{
    const KP q = bucket_select_kp(P, B, kb);
    unsigned char *w = (unsigned char *)ws;
    const size_t sel_b = align256(select_workspace_bytes(q, select_plan(q)));
    int32_t *tbl = (int32_t *)(w + sel_b);
    int32_t *tn = (int32_t *)(w + sel_b + align256((size_t)P.h_kv * (size_t)P.rows * (size_t)kb * sizeof(int32_t)));
    hipError_t e = launch_select(q, dtype, q_sel, B.centroid, nullptr, tbl, tn, w, st);
    if (e != hipSuccess)
        return e;
    bucket_expand_kernel<<<dim3((unsigned)P.rows, (unsigned)P.h_kv), dim3(256), 0, st>>>(P, B, tbl, tn, kb, idx, n_idx);
    return hipGetLastError();
}

} // namespace sa
