"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin is a plain function that raises AssertionError when the oracle
disagrees with what the mathematics or the pages fix:

  * closed forms of the pooling (constant keys, linear ramps, parallel keys),
    and numpy's mean as the textbook routine for full blocks;
  * brute-force enumeration of k-subsets for the selection rule (the best
    k-subset by total score, lexicographically smallest among equals, is the
    same set as "score descending, lower index first");
  * invariances of the group-summed score (head permutation, positive
    scaling, moving the whole group mass to one head);
  * torch's scaled_dot_product_attention in fp64 as an independent library for
    the two special cases that reduce to textbook attention: dense causal
    attention when k covers every candidate, and sink + sliding-window
    attention when k = 0;
  * Q = 0 (uniform weights: the output is the plain mean of V over the set,
    which fixes the set's size and forbids double counting) and V constant;
  * the S3R draft count |A| = keep + t + 1 for draft t;
  * hand-derived worked examples under tests/golden/;
  * overlapping pooling windows: ramp mid-points and token counts in closed
    form, and disjoint pooling again at overlap 0;
  * the group-score variants: a hand-worked two-head example whose three
    modes pick different blocks, one head (every mode ranks like the sum),
    the softmax scores summing to the group size, and a very large softmax
    temperature ranking like the sum.

``tests/test_oracle_mutants.py`` plants mistakes in copies of oracle.c and
checks that at least one of these pins fails for each.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import oracle
from workloads import (DTYPE_BF16, DTYPE_F32, POOL_L2SUM, POOL_MEAN, SELECT_ATTN, SELECT_MAX, SELECT_SOFTMAX,
                       SELECT_SUM, Workload, generate, small)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers

def wl(**kw) -> Workload:
    base = dict(name="pin", dtype=DTYPE_F32, h_q=2, h_kv=1, head_dim=4, seqlens_k=[16],
                seqlens_q=[16], block=2, pool=POOL_MEAN, topk=2, n_init=1, window=2)
    base.update(kw)
    return Workload(**base)


def cu(lens):
    return np.cumsum([0] + list(lens)).astype(np.int32)


def fixed_set(p_sel, n_init, window):
    return set(range(0, min(n_init, p_sel + 1))) | set(range(max(0, p_sel - window + 1), p_sel + 1))


def candidate_blocks(n, p_sel, n_init, window, g):
    F = fixed_set(p_sel, n_init, window)
    out = []
    for j in range(-(-n // g)):
        toks = set(range(j * g, min((j + 1) * g, n)))
        if max(toks) <= p_sel and not toks <= F:
            out.append(j)
    return out


def attended(p, p_sel, n_init, window, g, blocks):
    A = set(range(0, min(n_init, p + 1))) | set(range(max(0, p_sel - window + 1), p + 1))
    for j in blocks:
        A |= {t for t in range(j * g, (j + 1) * g) if t <= p}
    return A


def brute_topk(cands, score, k):
    kk = min(k, len(cands))
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(sorted(cands), kk):
        s = sum(score[j] for j in sub)
        if s > best_sum:                      # combinations come in lexicographic order:
            best, best_sum = sub, s           # keep the first (smallest) among equal sums
    return list(best) if best is not None else []


def positions(w, b):
    nk, nq = w.seqlens_k[b], w.seqlens_q[b]
    return list(range(nk - nq, nk))


def sdpa(q, k, v, mask, scale):
    """torch's fp64 attention; q [M, d], k/v [N, d], mask [M, N] bool."""
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None, None], k[None, None], v[None, None], attn_mask=mask[None, None], scale=scale)
    return o[0, 0]


# ------------------------------------------------------------------ compress

def pin_compress_constant_keys():
    """Keys constant within a (sequence, head) -> every pooled key equals that key."""
    w = wl(h_q=4, h_kv=2, head_dim=8, seqlens_k=[37, 64, 5], seqlens_q=[1, 1, 1], block=8)
    rng = np.random.default_rng(1)
    k = np.zeros((w.total_k, 2, 8), dtype=np.float32)
    c = cu(w.seqlens_k)
    vals = rng.standard_normal((3, 2, 8)).astype(np.float32)
    for b in range(3):
        k[c[b]:c[b + 1]] = vals[b]
    out = oracle.compress(w, k)
    for b in range(3):
        nb = -(-w.seqlens_k[b] // 8)
        for h in range(2):
            np.testing.assert_allclose(out[h, b, :nb], np.broadcast_to(vals[b, h], (nb, 8)),
                                       rtol=1e-14, atol=0)


def pin_compress_ramp_midpoint():
    """k_t = a + t*b -> pooled key of block j = a + (mid-point position of the block)*b."""
    g, n = 6, 45
    w = wl(h_q=1, h_kv=1, head_dim=3, seqlens_k=[n], seqlens_q=[1], block=g)
    a = np.array([1.0, -2.0, 0.5])
    bb = np.array([0.25, 1.0, -0.125])
    t = np.arange(n)[:, None]
    k = (a + t * bb).astype(np.float32)[:, None, :]
    out = oracle.compress(w, k)
    for j in range(-(-n // g)):
        t0, t1 = j * g, min((j + 1) * g, n) - 1
        np.testing.assert_allclose(out[0, 0, j], a + 0.5 * (t0 + t1) * bb, rtol=1e-13, atol=1e-13)


def pin_compress_numpy_mean():
    """Full blocks: numpy's mean over the block axis (bf16 inputs, exact widening)."""
    w = wl(dtype=DTYPE_BF16, h_q=8, h_kv=4, head_dim=16, seqlens_k=[128, 64], seqlens_q=[1, 1],
           block=16)
    x = generate(w)
    k = x["k"].float().numpy().astype(np.float64)
    out = oracle.compress(w, x["k"])
    c = cu(w.seqlens_k)
    for b in range(2):
        kb = k[c[b]:c[b + 1]].reshape(-1, 16, 4, 16).mean(axis=1)   # [nb, Hkv, d]
        np.testing.assert_allclose(out[:, b, :kb.shape[0]], kb.transpose(1, 0, 2), rtol=1e-12,
                                   atol=1e-14)


def pin_compress_l2sum():
    """L2SUM: parallel keys -> n * unit vector; any keys -> norm <= n; a zero key adds nothing."""
    g, d = 4, 8
    w = wl(h_q=1, h_kv=1, head_dim=d, seqlens_k=[4 * g + 2], seqlens_q=[1], block=g, pool=POOL_L2SUM)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((w.total_k, 1, d)).astype(np.float32)
    x = np.zeros(d, dtype=np.float32)
    x[:3] = [3.0, 4.0, 12.0]                 # norm 13
    for t in range(g):                       # block 0: positive multiples of x
        k[t, 0] = x * (t + 1)
    k[g + 1, 0] = 0.0                        # block 1: one zero key
    out = oracle.compress(w, k)
    np.testing.assert_allclose(out[0, 0, 0], g * x.astype(np.float64) / 13.0, rtol=1e-14, atol=1e-15)
    k1 = k[g:2 * g, 0].astype(np.float64)
    exp1 = sum(k1[i] / np.linalg.norm(k1[i]) for i in (0, 2, 3))
    np.testing.assert_allclose(out[0, 0, 1], exp1, rtol=1e-13, atol=1e-14)
    for j in range(out.shape[2]):
        n_j = min(g, w.total_k - j * g)
        assert np.linalg.norm(out[0, 0, j]) <= n_j + 1e-12
    assert abs(np.linalg.norm(out[0, 0, 0]) - g) < 1e-12          # equality for parallel keys


def pin_compress_overlap_closed_forms():
    """Windows [max(0, jg - o), e_j]: a ramp pools to the window's mid-point (MEAN), and
    positive multiples of one direction sum to the window's token count (L2SUM)."""
    g, n, o = 4, 23, 3
    a = np.array([1.0, -2.0, 0.5])
    bb = np.array([0.25, 1.0, -0.125])
    t = np.arange(n)[:, None]
    k = (a + t * bb).astype(np.float32)[:, None, :]
    w = wl(h_q=1, h_kv=1, head_dim=3, seqlens_k=[n], seqlens_q=[1], block=g, pool_overlap=o)
    out = oracle.compress(w, k)
    for j in range(-(-n // g)):
        t0, t1 = max(0, j * g - o), min((j + 1) * g, n) - 1
        np.testing.assert_allclose(out[0, 0, j], a + 0.5 * (t0 + t1) * bb, rtol=1e-13, atol=1e-13)
    kp = ((t + 1) * np.array([0.0, 2.0, 0.0])).astype(np.float32)[:, None, :]
    w2 = w.scaled(pool=POOL_L2SUM)
    out2 = oracle.compress(w2, kp)
    for j in range(-(-n // g)):
        cnt = min((j + 1) * g, n) - max(0, j * g - o)
        np.testing.assert_allclose(out2[0, 0, j], [0.0, cnt, 0.0], rtol=1e-14, atol=0)
    # overlap 0 is the disjoint pooling
    x = generate(wl(dtype=DTYPE_BF16, h_q=2, h_kv=1, head_dim=8, seqlens_k=[50], seqlens_q=[1], block=8))
    w3 = wl(dtype=DTYPE_BF16, h_q=2, h_kv=1, head_dim=8, seqlens_k=[50], seqlens_q=[1], block=8)
    np.testing.assert_array_equal(oracle.compress(w3, x["k"]), oracle.compress(w3.scaled(pool_overlap=0), x["k"]))


def _two_head_example(mode, tau=0.0, topk=1):
    """Token-level selection (g = 1) of one query at position 3 with heads q_0 = (1, 0),
    q_1 = (0, 1) over candidate keys (3, 0), (2, 2), (0, 2.5); token 3 is the window."""
    w = wl(h_q=2, h_kv=1, head_dim=2, seqlens_k=[4], seqlens_q=[1], block=1, topk=topk, n_init=0,
           window=1, select_mode=mode, select_tau=tau)
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]], dtype=np.float32)
    k = np.array([[[3.0, 0.0]], [[2.0, 2.0]], [[0.0, 2.5]], [[9.0, 9.0]]], dtype=np.float32)
    return oracle.select(w, q, None, k, want_scores=True)


def pin_select_modes_worked_example():
    """Per-head scores (3, 0), (2, 2), (0, 2.5): the sum ranks (4, 3, 2.5), the max (3, 2.5, 2);
    the softmax sum at tau = 1 is sum_h e^{l_hj} / sum_i e^{l_hi}."""
    r = _two_head_example(SELECT_SUM, topk=2)
    np.testing.assert_allclose(r["scores"][0, :3], np.array([3.0, 4.0, 2.5]) / math.sqrt(2), rtol=1e-14)
    assert list(r["idx"][0]) == [0, 1]
    r = _two_head_example(SELECT_MAX, topk=1)
    np.testing.assert_allclose(r["scores"][0, :3], np.array([3.0, 2.0, 2.5]) / math.sqrt(2), rtol=1e-14)
    assert list(r["idx"][0]) == [0]
    r = _two_head_example(SELECT_MAX, topk=2)
    assert list(r["idx"][0]) == [0, 2]
    l0, l1 = [3.0, 2.0, 0.0], [0.0, 2.0, 2.5]
    z0, z1 = sum(math.exp(x) for x in l0), sum(math.exp(x) for x in l1)
    want = [math.exp(l0[j]) / z0 + math.exp(l1[j]) / z1 for j in range(3)]
    r = _two_head_example(SELECT_SOFTMAX, tau=1.0, topk=2)
    np.testing.assert_allclose(r["scores"][0, :3], want, rtol=1e-13)
    assert list(r["idx"][0]) == [0, 2]
    r = _two_head_example(SELECT_SOFTMAX, tau=50.0, topk=1)     # nearly uniform: ranks like the sum
    assert list(r["idx"][0]) == [1]


def pin_select_modes_one_head():
    """One head per group: max over one head is that head, and a softmax is increasing in
    its logit, so every mode selects what the sum selects."""
    w = small("bf16_decode_32k").scaled(h_q=8, h_kv=8, topk=9)
    x = generate(w)
    kc = oracle.compress(w, x["k"])
    ref = oracle.select(w, x["q"], kc, x["k"])
    for mode, tau in ((SELECT_MAX, 0.0), (SELECT_SOFTMAX, 0.0), (SELECT_SOFTMAX, 0.3)):
        got = oracle.select(w.scaled(select_mode=mode, select_tau=tau), x["q"], kc, x["k"])
        np.testing.assert_array_equal(got["n"], ref["n"])
        np.testing.assert_array_equal(got["idx"], ref["idx"])


def pin_select_softmax_invariants():
    """Every head's softmax over the candidates sums to one, so the scores of a row sum to
    the group size; a very large temperature ranks like the sum of logits."""
    w = small("bf16_decode_32k").scaled(topk=6, select_mode=SELECT_SOFTMAX)
    x = generate(w)
    kc = oracle.compress(w, x["k"])
    r = oracle.select(w, x["q"], kc, x["k"], want_scores=True)
    tot = np.nansum(r["scores"], axis=1)
    ok = r["ncand"] > 0
    np.testing.assert_allclose(tot[ok], w.group, rtol=1e-12)
    big = oracle.select(w.scaled(select_tau=1e7), x["q"], kc, x["k"])
    ref = oracle.select(w.scaled(select_mode=SELECT_SUM), x["q"], kc, x["k"])
    np.testing.assert_array_equal(big["idx"], ref["idx"])


def pin_select_attn_uniform_queries():
    """Q = 0: every query spreads its mass evenly over its p_i + 1 visible tokens, so
    block j scores sum_i G |block j| / (p_i + 1) (shared rows: 6 drafts)."""
    g, n_hist, m = 3, 40, 6
    w = wl(h_q=4, h_kv=2, head_dim=8, seqlens_k=[n_hist + m, 29 + m], seqlens_q=[m, m], block=g, topk=5,
           n_init=2, window=4, shared_selection=1, select_mode=SELECT_ATTN)
    x = generate(w.scaled(dtype=DTYPE_F32))
    q = torch.zeros_like(x["q"])
    r = oracle.select(w, q, None, x["k"], want_scores=True)
    for rr, b in enumerate(r["rows"]):
        nk = w.seqlens_k[b]
        q0 = nk - m
        for j in range(-(-nk // g)):
            s = r["scores"][rr, j]
            if np.isnan(s):
                continue
            size = min((j + 1) * g, nk) - j * g
            want = sum(w.group * size / (q0 + t + 1) for t in range(m))
            assert abs(s - want) < 1e-12 * want, (b, j, s, want)


def pin_select_attn_worked_example():
    """One query at position 2, one head, keys with logits (ln 4, 0, ln 3) over sqrt(d) = 1
    (d = 1): masses 4/8, 1/8, 3/8 of which tokens 0 and 1 are candidates (window 1)."""
    w = wl(h_q=1, h_kv=1, head_dim=1, seqlens_k=[3], seqlens_q=[1], block=1, topk=1, n_init=0, window=1,
           select_mode=SELECT_ATTN)
    q = torch.tensor([[[1.0]]], dtype=torch.float32)
    k = torch.tensor([[[math.log(4.0)]], [[0.0]], [[math.log(3.0)]]], dtype=torch.float32)
    r = oracle.select(w, q, None, k, want_scores=True)
    kf = k.double().numpy().reshape(-1)
    z = np.exp(kf).sum()
    np.testing.assert_allclose(r["scores"][0, :2], np.exp(kf[:2]) / z, rtol=1e-14)
    assert list(r["idx"][0]) == [0]
    np.testing.assert_allclose(np.exp(kf) / z, [0.5, 0.125, 0.375], rtol=1e-6)


def pin_select_attn_shift_invariance():
    """Adding to every key a vector orthogonal to every query leaves every softmax, hence
    every mass and the selection, unchanged."""
    w = wl(dtype=DTYPE_F32, h_q=2, h_kv=1, head_dim=8, seqlens_k=[70], seqlens_q=[3], block=2, topk=6,
           n_init=1, window=5, shared_selection=1, select_mode=SELECT_ATTN)
    x = generate(w)
    q = x["q"].clone()
    q[..., 7] = 0.0                            # every query lies in the first 7 dimensions
    k2 = x["k"].clone()
    k2[..., 7] += 3.0                          # so this shift is orthogonal to all of them
    a = oracle.select(w, q, None, x["k"], want_scores=True)
    b = oracle.select(w, q, None, k2, want_scores=True)
    np.testing.assert_allclose(b["scores"], a["scores"], rtol=1e-12, atol=0)
    np.testing.assert_array_equal(a["idx"], b["idx"])


def pin_select_attn_one_query_ranks_by_dot():
    """One query and one head per row: exp(l_t - lse) is increasing in the logit, so the
    selection is the dot-product selection (g = 1)."""
    w = wl(dtype=DTYPE_BF16, h_q=3, h_kv=3, head_dim=16, seqlens_k=[300, 123], seqlens_q=[1, 1], block=1,
           topk=17, n_init=4, window=8)
    x = generate(w)
    ref = oracle.select(w, x["q"], None, x["k"])
    got = oracle.select(w.scaled(select_mode=SELECT_ATTN), x["q"], None, x["k"])
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["n"], ref["n"])


def _bucket_index(points, C, NB, cap, g=1):
    """Bucket index of one sequence, one KV head, from given pooled keys [n, d] (fp64)."""
    pts = np.asarray(points, dtype=np.float64)
    w = wl(h_q=1, h_kv=1, head_dim=pts.shape[1], seqlens_k=[pts.shape[0] * g], seqlens_q=[1], block=g,
           bucket_block=C, bucket_count=NB, bucket_cap=cap)
    return w, oracle.bucket_build(w, pts[None, None])


def _buckets(ix, blk=0):
    mem, off = ix["member"][0, 0, blk], ix["offset"][0, 0, blk]
    return [sorted(mem[off[i]:off[i + 1]].tolist()) for i in range(len(off) - 1)]


def pin_bucket_pairs_and_centroids():
    """Four well separated pairs: each pair is each other's cheapest merge; centroids are
    the normalised pair sums."""
    pts = [(0, 5), (1, 5), (10, 0), (11, 0), (0, -10), (1, -10), (-20, 0), (-21, 0)]
    w, ix = _bucket_index(pts, C=8, NB=4, cap=4)
    assert _buckets(ix) == [[0, 1], [2, 3], [4, 5], [6, 7]]
    for i, (a, b) in enumerate([(0, 1), (2, 3), (4, 5), (6, 7)]):
        s = np.add(pts[a], pts[b]).astype(np.float64)
        np.testing.assert_allclose(ix["centroid"][0, 0, 0, i], s / np.linalg.norm(s), rtol=1e-7)


def pin_bucket_truncation_by_cost_then_name():
    """Four mutual pairs but NB = 5 leaves room for three merges: the cheapest (Ward cost
    0.125) and, of the three tied at 0.5, the two with the lower names."""
    pts = [(0, 0), (1, 0), (20, 0), (20.5, 0), (40, 0), (41, 0), (60, 0), (61, 0)]
    pts = [(x, 100.0) for x, _ in pts]
    w, ix = _bucket_index(pts, C=8, NB=5, cap=4)
    assert _buckets(ix) == [[0, 1], [2, 3], [4, 5], [6], [7]]
    assert list(ix["offset"][0, 0, 0]) == [0, 2, 4, 6, 7, 8]


def pin_bucket_ward_weighting():
    """Point 2 at 0 is nearer to the centroid of the pair {0, 1} (at -2.8) than to point 3
    (at 3), but Ward's cost n_A n_B / (n_A + n_B) d^2 is 5.23 against 4.5: it joins point 3."""
    pts = [(-3.0, 1.0), (-2.6, 1.0), (0.0, 1.0), (3.0, 1.0)]
    w, ix = _bucket_index(pts, C=4, NB=2, cap=4)             # {0, 1, 2} would fit
    assert _buckets(ix) == [[0, 1], [2, 3]]


def pin_bucket_ward_uses_means():
    """Ward's cost compares bucket means: after {0, 1} merges (mean 10.1), point 2 at 11
    costs 2/3 * 0.9^2 = 0.54 to join it and point 3 at 19 costs 32 to join point 2, so
    {0, 1, 2} forms; comparing member sums (20.2) instead would pair {0, 1} with point 3."""
    pts = [(10.0, 0.0), (10.2, 0.0), (11.0, 0.0), (19.0, 0.0)]
    w, ix = _bucket_index(pts, C=4, NB=2, cap=4)
    assert _buckets(ix) == [[0, 1, 2], [3]]


def pin_bucket_invariants():
    """Random keys: each complete cluster block is partitioned into exactly NB buckets of at
    most cap/g groups, named and listed in order; centroids are normalised member sums;
    the incomplete last block has no buckets."""
    g, C, NB, cap = 4, 64, 8, 16
    w = wl(dtype=DTYPE_BF16, h_q=4, h_kv=2, head_dim=16, seqlens_k=[3 * C + 37, 2 * C], seqlens_q=[1, 1],
           block=g, pool=POOL_L2SUM, bucket_block=C, bucket_count=NB, bucket_cap=cap)
    x = generate(w)
    kc = oracle.compress(w, x["k"])
    ix = oracle.bucket_build(w, kc)
    M = C // g
    for c in range(2):
        for b, nk in enumerate(w.seqlens_k):
            for blk in range(ix["member"].shape[2]):
                mem, off = ix["member"][c, b, blk], ix["offset"][c, b, blk]
                if (blk + 1) * C > nk:
                    assert (mem == -1).all() and (off == 0).all()
                    continue
                assert sorted(mem.tolist()) == list(range(M))
                sizes = np.diff(off)
                assert len(sizes) == NB and (sizes >= 1).all() and (sizes <= cap // g).all()
                names = [mem[off[i]] for i in range(NB)]
                assert names == sorted(names)
                for i in range(NB):
                    grp = mem[off[i]:off[i + 1]]
                    assert list(grp) == sorted(grp)
                    ssum = kc[c, b, blk * M + grp].astype(np.float32).astype(np.float64).sum(0)
                    np.testing.assert_allclose(ix["centroid"][c, b, blk, i], ssum / np.linalg.norm(ssum),
                                               rtol=1e-5, atol=1e-6)


def pin_bucket_select():
    """kb >= every visible bucket selects every group of the complete cluster blocks that
    end at or before p_sel, except those wholly inside the sink or window; kb = 1 with the
    query along one centroid takes that bucket."""
    g, C, NB, cap = 4, 64, 8, 16
    w = wl(dtype=DTYPE_F32, h_q=2, h_kv=1, head_dim=16, seqlens_k=[5 * C + 10], seqlens_q=[40], block=g,
           pool=POOL_L2SUM, n_init=6, window=40, bucket_block=C, bucket_count=NB, bucket_cap=cap,
           bucket_topk=1000)
    x = generate(w)
    ix = oracle.bucket_build(w, oracle.compress(w, x["k"]))
    r = oracle.bucket_select(w, x["q"], ix)
    for rr in range(w.rows):
        p = w.seqlens_k[0] - w.seqlens_q[0] + rr
        ncb = (p + 1) // C
        hi = p - w.window + 1                    # groups wholly in the sink or window are left out
        want = [j for j in range(ncb * C // g) if j * g < hi and (j + 1) * g > w.n_init]
        assert r["idx"][rr, :r["n"][rr]].tolist() == want
    # one bucket: a query along the centroid of bucket 5 of block 2 (unit centroids: it wins)
    w1 = w.scaled(bucket_topk=1, seqlens_q=[1], seqlens_k=[4 * C])
    target = ix["centroid"][0, 0, 2, 5]
    q = torch.zeros((1, 2, 16), dtype=torch.float32)
    q[0, 0] = torch.from_numpy(target * 3.0).float()
    r1 = oracle.bucket_select(w1, q, ix)
    mem, off = ix["member"][0, 0, 2], ix["offset"][0, 0, 2]
    want = sorted((2 * (C // g) + mem[off[5]:off[6]]).tolist())
    assert r1["idx"][0, :r1["n"][0]].tolist() == want and r1["nbk"][0] == 1


# ------------------------------------------------------------------ select

def _planted_scores_case(rng, g, n, pool, n_init, window, topk, G=2, d=8, n_levels=4):
    """Keys whose pooled dim-0 equals a chosen level a_j; queries that sum to (sigma, 0, ...)."""
    w = wl(h_q=G, h_kv=1, head_dim=d, seqlens_k=[n], seqlens_q=[n], block=g, pool=pool,
           topk=topk, n_init=n_init, window=window)
    nb = -(-n // g)
    levels = rng.integers(-n_levels, n_levels + 1, size=nb).astype(np.float64)
    k = rng.standard_normal((n, 1, d)).astype(np.float32)
    for j in range(nb):
        k[j * g:(j + 1) * g, 0, 0] = levels[j]
    q = np.zeros((n, G, d), dtype=np.float32)
    sigma = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
    r = rng.standard_normal((n, d)).astype(np.float32)
    r[:, 0] = 0
    q[:, 0, :] = r
    q[:, 1, :] = -r                          # cancels exactly in the group sum
    q[:, 0, 0] = sigma * 0.75
    q[:, 1, 0] = sigma * 0.25
    return w, q, k, levels


def pin_select_bruteforce():
    """Selection == brute-force best k-subset (ties -> lexicographically smallest)."""
    rng = np.random.default_rng(3)
    cases = 0
    for g, n, n_init, window, topk in [(1, 12, 0, 2, 3), (2, 19, 1, 2, 2), (3, 23, 2, 4, 4),
                                       (2, 24, 0, 1, 3), (4, 30, 3, 5, 1), (1, 10, 2, 1, 4),
                                       (3, 20, 0, 3, 0), (2, 16, 4, 4, 8)]:
        w, q, k, levels = _planted_scores_case(rng, g, n, POOL_MEAN, n_init, window, topk)
        kc = oracle.compress(w, k) if g > 1 else None
        sel = oracle.select(w, q, kc, k)
        for p in range(n):
            C = candidate_blocks(n, p, n_init, window, g)
            want = brute_topk(C, {j: levels[j] for j in C}, topk)
            got = list(sel["idx"][p, :sel["n"][p]])
            assert got == want, (g, n, n_init, window, topk, p, got, want)
            assert all(x == -1 for x in sel["idx"][p, sel["n"][p]:])
            assert sel["ncand"][p] == len(C)
            cases += 1
    assert cases > 100


def pin_select_l2sum_order():
    """L2SUM pooling: block of keys lambda_t*(a_j, 1, 0..) -> ranking follows a_j."""
    rng = np.random.default_rng(4)
    g, n, d = 4, 64, 8
    w = wl(h_q=1, h_kv=1, head_dim=d, seqlens_k=[n], seqlens_q=[1], block=g, pool=POOL_L2SUM,
           topk=5, n_init=4, window=8)
    nb = n // g
    a = rng.permutation(np.linspace(-3, 3, nb))
    k = np.zeros((n, 1, d), dtype=np.float32)
    for j in range(nb):
        for t in range(j * g, (j + 1) * g):
            lam = rng.uniform(0.5, 3.0)
            k[t, 0, 0] = lam * a[j]
            k[t, 0, 1] = lam
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 1.0
    sel = oracle.select(w, q, oracle.compress(w, k), k)
    C = candidate_blocks(n, n - 1, 4, 8, g)
    want = sorted(sorted(C, key=lambda j: -a[j])[:5])
    assert list(sel["idx"][0, :sel["n"][0]]) == want


def pin_select_equal_scores():
    """All pooled keys equal -> the k lowest-index candidates."""
    w = wl(h_q=4, h_kv=2, head_dim=8, seqlens_k=[200, 97], seqlens_q=[3, 2], block=8, topk=5,
           n_init=8, window=16)
    rng = np.random.default_rng(5)
    k = np.broadcast_to(rng.standard_normal((1, 2, 8)), (w.total_k, 2, 8)).astype(np.float32).copy()
    q = rng.standard_normal((w.total_q, 4, 8)).astype(np.float32)
    sel = oracle.select(w, q, oracle.compress(w, k), k)
    for r, (row, h) in enumerate(zip(sel["rows"], sel["heads"])):
        b = 0 if row < 3 else 1
        p = positions(w, b)[row - (0 if b == 0 else 3)]
        C = candidate_blocks(w.seqlens_k[b], p, 8, 16, 8)
        assert list(sel["idx"][r, :sel["n"][r]]) == C[:5], (row, h)


def pin_select_invariances():
    """Group-summed score: head permutation, positive scaling and moving all the
    group's query mass onto one head leave the selection unchanged (integer
    data, so every sum is exact)."""
    rng = np.random.default_rng(6)
    w = wl(dtype=DTYPE_BF16, h_q=8, h_kv=2, head_dim=16, seqlens_k=[300, 180], seqlens_q=[40, 7],
           block=8, topk=6, n_init=8, window=24)
    k = torch.tensor(rng.integers(-4, 5, size=(w.total_k, 2, 16)), dtype=torch.bfloat16)
    q = torch.tensor(rng.integers(-3, 4, size=(w.total_q, 8, 16)), dtype=torch.bfloat16)
    kc = oracle.compress(w, k)
    ref = oracle.select(w, q, kc, k)
    perm = torch.tensor([2, 0, 3, 1, 7, 5, 4, 6])     # permutes within each group of 4
    for q2 in (q[:, perm].contiguous(),
               (q.float() * 4).to(torch.bfloat16),
               torch.cat([q.float().view(-1, 2, 4, 16).sum(2, keepdim=True),
                          torch.zeros(w.total_q, 2, 3, 16)], 2).view(-1, 8, 16).to(torch.bfloat16)):
        got = oracle.select(w, q2, kc, k)
        np.testing.assert_array_equal(got["idx"], ref["idx"])
        np.testing.assert_array_equal(got["n"], ref["n"])
    # swapping the two groups' heads swaps the two KV heads' selections
    qs = torch.cat([q[:, 4:], q[:, :4]], 1).contiguous()
    ks = torch.cat([k[:, 1:], k[:, :1]], 1).contiguous()
    got = oracle.select(w, qs, oracle.compress(w, ks), ks)
    n_rows = w.rows
    np.testing.assert_array_equal(got["idx"][:n_rows], ref["idx"][n_rows:])


# ------------------------------------------------------------------ attend

def _rand_case(seed, dtype, **kw):
    w = wl(dtype=dtype, **kw)
    x = generate(w.scaled(seed=seed))
    return w, x


def _f64(t):
    return t.double() if isinstance(t, torch.Tensor) else torch.tensor(t, dtype=torch.float64)


def pin_attend_dense_when_k_covers():
    """k >= |C| (and w >= g) -> dense causal attention (torch fp64 SDPA)."""
    for dtype, kw in [(DTYPE_F32, dict(h_q=4, h_kv=2, head_dim=16, seqlens_k=[70, 33],
                                       seqlens_q=[70, 5], block=8, topk=100, n_init=3, window=8)),
                      (DTYPE_BF16, dict(h_q=2, h_kv=1, head_dim=32, seqlens_k=[129], seqlens_q=[40],
                                        block=4, topk=64, n_init=0, window=5))]:
        w, x = _rand_case(11, dtype, **kw)
        r = oracle.run(w, x)
        scale = 1 / math.sqrt(w.head_dim)
        c = cu(w.seqlens_k)
        cq = cu(w.seqlens_q)
        G = w.group
        for b in range(w.batch):
            pos = torch.tensor(positions(w, b))
            mask = torch.arange(w.seqlens_k[b])[None, :] <= pos[:, None]
            for h in range(w.h_q):
                o = sdpa(_f64(x["q"][cq[b]:cq[b + 1], h]), _f64(x["k"][c[b]:c[b + 1], h // G]),
                         _f64(x["v"][c[b]:c[b + 1], h // G]), mask, scale)
                sel = (r["reqs"] >= cq[b]) & (r["reqs"] < cq[b + 1]) & (r["heads"] == h)
                np.testing.assert_allclose(r["out"][sel], o.numpy(), rtol=1e-12, atol=1e-12)


def pin_attend_sink_window_when_k_zero():
    """k = 0 -> attention with sink tokens and a sliding window (torch fp64 SDPA, band mask)."""
    w, x = _rand_case(12, DTYPE_BF16, h_q=4, h_kv=1, head_dim=16, seqlens_k=[90, 61],
                      seqlens_q=[90, 20], block=4, topk=0, n_init=5, window=9)
    r = oracle.run(w, x)
    scale = 1 / math.sqrt(w.head_dim)
    c, cq = cu(w.seqlens_k), cu(w.seqlens_q)
    for b in range(w.batch):
        pos = torch.tensor(positions(w, b))[:, None]
        t = torch.arange(w.seqlens_k[b])[None, :]
        mask = (t <= pos) & ((t < 5) | (t >= pos - 9 + 1))
        for h in range(w.h_q):
            o = sdpa(_f64(x["q"][cq[b]:cq[b + 1], h]), _f64(x["k"][c[b]:c[b + 1], 0]),
                     _f64(x["v"][c[b]:c[b + 1], 0]), mask, scale)
            sel = (r["reqs"] >= cq[b]) & (r["reqs"] < cq[b + 1]) & (r["heads"] == h)
            np.testing.assert_allclose(r["out"][sel], o.numpy(), rtol=1e-12, atol=1e-12)


def pin_attend_zero_query_is_set_mean():
    """Q = 0 -> uniform weights: O = plain mean of V over init U window U selected blocks."""
    w, x = _rand_case(13, DTYPE_F32, h_q=2, h_kv=1, head_dim=8, seqlens_k=[150, 77],
                      seqlens_q=[150, 9], block=8, topk=3, n_init=6, window=11)
    kc = oracle.compress(w, x["k"])
    idx, n = oracle.table(w, oracle.select(w, x["q"], kc, x["k"]))     # selection from real Q
    att = oracle.attend(w, torch.zeros_like(x["q"]), x["k"], x["v"], idx, n)
    c, cq = cu(w.seqlens_k), cu(w.seqlens_q)
    v = x["v"].double().numpy()
    for r, (i, h) in enumerate(zip(att["reqs"], att["heads"])):
        b = 0 if i < cq[1] else 1
        p = positions(w, b)[i - cq[b]]
        blocks = list(idx[0, i, :n[0, i]])
        for j in blocks:                                           # selected: fully visible
            assert (j + 1) * 8 - 1 <= p
        A = attended(p, p, 6, 11, 8, blocks)
        assert att["count"][r] == len(A)
        assert set(range(0, min(6, p + 1))) <= A                  # init contained
        assert set(range(max(0, p - 10), p + 1)) <= A              # window contained
        want = v[[c[b] + t for t in sorted(A)], 0].mean(0)
        np.testing.assert_allclose(att["out"][r], want, rtol=1e-12, atol=1e-13)


def pin_attend_constant_v():
    """V rows all equal -> O is that row for any query (weights sum to one)."""
    w, x = _rand_case(14, DTYPE_BF16, h_q=4, h_kv=2, head_dim=16, seqlens_k=[100],
                      seqlens_q=[100], block=4, topk=5, n_init=2, window=7)
    row = torch.randn(2, 16).to(torch.bfloat16)
    x["v"] = row[None].expand(100, 2, 16).contiguous()
    r = oracle.run(w, x)
    want = row.double().numpy()[r["heads"] // 2]
    np.testing.assert_allclose(r["out"], want, rtol=1e-13, atol=1e-14)


def pin_draft_counts():
    """Shared selection (S3R drafts): one set per sequence; draft t attends keep + t + 1 tokens."""
    w = small("bf16_draft_decode")
    x = generate(w)
    r = oracle.run(w, x)
    cq = cu(w.seqlens_q)
    for b in range(w.batch):
        keep = w.topk_per_seq[b] + w.window
        for t in range(w.seqlens_q[b]):
            sel = (r["reqs"] == cq[b] + t)
            assert np.all(r["count"][sel] == keep + t + 1), (b, t, r["count"][sel], keep)
        assert np.all(r["n_idx"][:, b] == w.topk_per_seq[b])


def pin_golden_hand_examples():
    """Hand-derived worked examples (tests/golden/hand_examples.json)."""
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        w = Workload(name=case["name"], dtype=DTYPE_F32, pool=POOL_MEAN, **case["workload"])
        q = np.array(case["q"], dtype=np.float32)
        k = np.array(case["k"], dtype=np.float32)
        v = np.array(case["v"], dtype=np.float32)
        kc = oracle.compress(w, k) if w.block > 1 else None
        if kc is not None:
            np.testing.assert_allclose(kc[0, 0, :len(case["k_cmp"])], case["k_cmp"], rtol=0, atol=0)
        sel = oracle.select(w, q, kc, k)
        assert [list(map(int, s[:n])) for s, n in zip(sel["idx"], sel["n"])] == case["selected"]
        np.testing.assert_allclose(sel["sk"], case["s_k"], rtol=1e-14)
        np.testing.assert_allclose(sel["sk1"], case["s_k1"], rtol=1e-14)
        idx, n = oracle.table(w, sel)
        att = oracle.attend(w, q, k, v, idx, n)
        assert list(att["count"]) == case["count"]
        np.testing.assert_allclose(att["out"], case["out"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(att["lse"], case["lse"], rtol=1e-13)


def pin_empty_and_ragged():
    """No candidates (short sequence): nothing selected, attention = init + window only;
    ragged last block: the partial block is never a candidate while it is not wholly visible."""
    w, x = _rand_case(15, DTYPE_F32, h_q=2, h_kv=1, head_dim=8, seqlens_k=[10, 29],
                      seqlens_q=[1, 29], block=8, topk=4, n_init=8, window=8)
    r = oracle.run(w, x)
    assert r["n_idx"][0, 0] == 0                         # seq 0: p = 9, non-F tokens = [8, 2): none
    assert r["count"][0] == 10 and r["count"][1] == 10
    for i in range(29):                                  # seq 1: block 3 = tokens 24..28 (ragged)
        row = 1 + i
        assert 3 not in r["idx"][0, row, :r["n_idx"][0, row]] or i >= 28


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
