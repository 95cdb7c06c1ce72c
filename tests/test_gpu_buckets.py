"""The LSA flat bucket index through the C ABI against the oracle (needs an MI355X).

Build: every complete cluster block's partition into buckets must equal the
oracle's, except in blocks where the oracle saw a near-tied decision (relative
margin < 1e-4): the oracle decides its merges in fp64 and the kernel in fp32,
each from pooled keys it computes itself, so a near tie may go either way.  Centroids of
equal partitions agree to fp32 rounding.  Retrieval: rows whose visible blocks all
partition alike must select the oracle's groups (or sit on a bucket-score near
tie).  Attention runs on the GPU's table and is compared with the oracle's
attention on that same table.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import DTYPE_BF16, FULL, POOL_L2SUM, POOL_MEAN, Workload, generate, small

pytestmark = pytest.mark.gpu

MARGIN = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _width(w):
    return w.bucket_topk * (w.bucket_cap // w.block)


def _partition(member, offset):
    return [tuple(member[offset[i]:offset[i + 1]].tolist()) for i in range(len(offset) - 1)]


def _check_build(w, gx, ox):
    """Returns the set of (head, sequence, block) whose partitions differ (all near-tied)."""
    gm, go, gc = gx.member.cpu().numpy(), gx.offset.cpu().numpy(), gx.centroid.cpu().numpy()
    diff = set()
    for c in range(w.h_kv):
        for b, nk in enumerate(w.seqlens_k):
            for blk in range(ox["member"].shape[2]):
                if (blk + 1) * w.bucket_block > nk:
                    assert (gm[c, b, blk] == -1).all()
                    continue
                if _partition(gm[c, b, blk], go[c, b, blk]) != _partition(ox["member"][c, b, blk],
                                                                          ox["offset"][c, b, blk]):
                    assert ox["margin"][c, b, blk] < MARGIN, (c, b, blk, ox["margin"][c, b, blk])
                    diff.add((c, b, blk))
                    continue
                np.testing.assert_allclose(gc[c, b, blk], ox["centroid"][c, b, blk], rtol=0, atol=2e-6)
    return diff


def _check_select(w, x, ox, idx, n_idx, diff, rows=None, heads=None):
    sel = oracle.bucket_select(w, x["q"], ox, rows=rows, heads=heads)
    compared = 0
    for r, (row, c) in enumerate(zip(sel["rows"], sel["heads"])):
        b = row if w.shared_selection else int(np.searchsorted(np.cumsum(w.seqlens_q), row, side="right"))
        q0 = w.seqlens_k[b] - w.seqlens_q[b]
        p_sel = q0 - 1 if w.shared_selection else q0 + row - int(np.sum(w.seqlens_q[:b]))
        vis = min((p_sel + 1) // w.bucket_block, w.seqlens_k[b] // w.bucket_block)
        if any((c, b, blk) in diff for blk in range(vis)):
            continue
        compared += 1
        got = idx[c, row, :n_idx[c, row]].tolist()
        want = sel["idx"][r, :sel["n"][r]].tolist()
        if got == want:
            assert all(v == -1 for v in idx[c, row, n_idx[c, row]:])
            continue
        sk, sk1, fl = sel["sk"][r], sel["sk1"][r], sel["floor"][r]
        tie = not np.isnan(sk1) and (abs(sk - sk1) < 1e-4 * max(abs(sk), abs(sk1)) or abs(sk - sk1) < fl)
        assert tie, (row, c, got[:8], want[:8], sk, sk1)
    return compared


def _run(w, x, xg):
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"])
    gx = sa.bucket_build(p, kc, sa.BucketIndex(p, w.bucket_block, w.bucket_count, w.bucket_cap))
    idx, n_idx = sa.bucket_select(p, xg["q"], gx, w.bucket_topk)
    out, lse = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx, want_lse=True)
    torch.cuda.synchronize()
    return p, gx, idx.cpu().numpy(), n_idx.cpu().numpy(), out, lse


SHAPES = {
    # the 1M chunk's index shape at small size: 512-token blocks of 128 groups of 4, 64 buckets
    "lsa_chunk": lambda: small("bf16_chunked_prefill_1m").scaled(bucket_topk=32),
    # several sequences and KV heads, 32 groups of 8 tokens per block, mean pooling, d 64
    "multi_head": lambda: Workload(name="bkt", dtype=DTYPE_BF16, h_q=8, h_kv=2, head_dim=64,
                                   seqlens_k=[3000, 1500, 700], seqlens_q=[1, 1, 1], block=8, pool=POOL_MEAN,
                                   topk=1, n_init=8, window=64, seed=91, bucket_block=256, bucket_count=16,
                                   bucket_cap=32, bucket_topk=5),
    # 15 groups per cluster block (not a multiple of the 8 lanes a bucket's searches use)
    "odd_groups": lambda: Workload(name="bkt3", dtype=DTYPE_BF16, h_q=8, h_kv=2, head_dim=128,
                                   seqlens_k=[2400, 1100], seqlens_q=[1, 1], block=4, pool=POOL_MEAN,
                                   topk=1, n_init=4, window=64, seed=93, bucket_block=60, bucket_count=8,
                                   bucket_cap=16, bucket_topk=6),
    # 6 groups per cluster block (fewer than those 8 lanes)
    "few_groups": lambda: Workload(name="bkt4", dtype=DTYPE_BF16, h_q=4, h_kv=1, head_dim=64,
                                   seqlens_k=[1500, 800], seqlens_q=[1, 1], block=4, pool=POOL_MEAN,
                                   topk=1, n_init=4, window=32, seed=94, bucket_block=24, bucket_count=3,
                                   bucket_cap=16, bucket_topk=5),
    # per-query rows of a prefill chunk, L2SUM, drafts-style shared rows off
    "prefill_rows": lambda: Workload(name="bkt2", dtype=DTYPE_BF16, h_q=4, h_kv=1, head_dim=128,
                                     seqlens_k=[6000], seqlens_q=[700], block=4, pool=POOL_L2SUM, topk=1, n_init=4,
                                     window=512, seed=92, bucket_block=512, bucket_count=64, bucket_cap=16,
                                     bucket_topk=12),
}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_bucket_index_and_retrieval(shape):
    w = SHAPES[shape]()
    w = w.scaled(topk=_width(w))
    x, xg = parity.gen_pair(w)
    p, gx, idx, n_idx, out, lse = _run(w, x, xg)
    ox = oracle.bucket_build(w, oracle.compress(w, x["k"]))
    diff = _check_build(w, gx, ox)
    n_cmp = _check_select(w, x, ox, idx, n_idx, diff)
    assert n_cmp >= (w.rows * w.h_kv) // 2
    att = oracle.attend(w, x["q"], x["k"], x["v"], idx, n_idx)
    parity.check_output(w, out.float().cpu().reshape(-1, w.head_dim), att["out"])
    assert np.abs(lse.cpu().t().reshape(-1).double().numpy() - att["lse"]).max() < parity.lse_tol(w)


@pytest.mark.parametrize("plan", ["1", "5"])
def test_bucket_decode_rows_both_plans(plan, monkeypatch):
    """One query per sequence: the centroid scores of a row are ranked by the part + merge
    plan ("1") and by the one-workgroup-per-row plan ("5") alike."""
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", plan)
    w = SHAPES["multi_head"]()
    w = w.scaled(topk=_width(w))
    x, xg = parity.gen_pair(w)
    p, gx, idx, n_idx, out, lse = _run(w, x, xg)
    ox = oracle.bucket_build(w, oracle.compress(w, x["k"]))
    diff = _check_build(w, gx, ox)
    assert _check_select(w, x, ox, idx, n_idx, diff) >= (w.rows * w.h_kv) // 2


def test_full_chunked_prefill_1m_buckets_sampled():
    """The 1M chunk with the LSA bucket index: 2048 cluster blocks clustered, 256 buckets
    (about 2048 keys) per query; sampled rows and requests against the oracle."""
    w = FULL["bf16_chunked_prefill_1m"]().scaled(bucket_topk=256)
    w = w.scaled(topk=_width(w))
    xg = generate(w, device="cuda")
    p, gx, idx, n_idx, out, lse = _run(w, None, xg)
    x = {k: (t.cpu() if isinstance(t, torch.Tensor) else t) for k, t in xg.items()}
    ox = oracle.bucket_build(w, oracle.compress(w, x["k"]))
    diff = _check_build(w, gx, ox)
    assert len(diff) <= 16
    rng = np.random.default_rng(21)
    rows = rng.choice(w.rows, size=24, replace=False)
    _check_select(w, x, ox, idx, n_idx, diff, rows=rows, heads=np.zeros(len(rows), dtype=np.int32))
    reqs = rng.choice(w.total_q, size=128, replace=False)
    hs = rng.integers(0, w.h_q, size=len(reqs))
    att = oracle.attend(w, x["q"], x["k"], x["v"], idx, n_idx, reqs=reqs, heads=hs)
    gout = out.float().cpu().reshape(w.total_q, w.h_q, w.head_dim)[reqs, hs].double().numpy()
    parity.check_output(w, gout, att["out"])


def test_incremental_build():
    """Building from block f rewrites blocks f.. exactly as a full build and leaves the
    earlier blocks untouched (a chunk stream clusters each block once)."""
    w = SHAPES["lsa_chunk"]()
    w = w.scaled(topk=_width(w))
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"])
    full = sa.bucket_build(p, kc, sa.BucketIndex(p, w.bucket_block, w.bucket_count, w.bucket_cap))
    part = sa.BucketIndex(p, w.bucket_block, w.bucket_count, w.bucket_cap)
    part.member.fill_(-7)
    part.offset.fill_(-7)
    part.centroid.fill_(7.0)
    f = 20
    sa.bucket_build(p, kc, part, build_from=f)
    torch.cuda.synchronize()
    assert (part.member[:, :, :f] == -7).all() and (part.offset[:, :, :f] == -7).all()
    assert (part.centroid[:, :, :f] == 7.0).all()
    assert torch.equal(part.member[:, :, f:], full.member[:, :, f:])
    assert torch.equal(part.offset[:, :, f:], full.offset[:, :, f:])
    assert torch.equal(part.centroid[:, :, f:], full.centroid[:, :, f:])
