"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Small workloads: every row and every (query, head) compared.  Full-size
workloads: the launch configuration the benchmark times, compared on sampled
rows and requests the oracle computes one by one; the two prefill workloads
also have every one of their selections compared.  Edge cases: k = 0, k >=
|C| (dense), no sink, sequences with no candidates, ragged tails, head_dim
64, GQA group 1, explicit query offsets.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import DTYPE_BF16, DTYPE_F32, FULL, POOL_L2SUM, POOL_MEAN, Workload, generate, small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name", list(FULL))
def test_small_workload_parity(name):
    w = small(name)
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_tiny_fp32_prefill_full():
    w = FULL["tiny_fp32_prefill"]()
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


EDGE = {
    "k0": dict(topk=0),
    "dense": dict(topk=4096),
    "no_sink": dict(n_init=0),
    "wide_window": dict(window=1000),
    "odd_block": dict(block=7, topk=5, n_init=3, window=9),
    "d64_bf16": dict(head_dim=64),
    "group1": dict(h_q=8, h_kv=8),
    "l2sum": dict(pool=POOL_L2SUM, block=4, topk=9),
    # multi-query union tiles (per-query selection, block a multiple of 32)
    "tile_d64": dict(head_dim=64, block=32, topk=7),
    "tile_g16": dict(h_q=16, h_kv=1, block=32, topk=5, n_init=0, window=33),
    # LDS-shared 64-token tiles (block 64, a sequence of >= 256 queries)
    "wg_g4": dict(block=64, topk=5),
    "wg_g8": dict(h_q=16, h_kv=2, block=64, topk=4, n_init=64, window=100),
    "wg_g16_window1": dict(h_q=16, h_kv=1, block=64, topk=3, n_init=0, window=1),
}


@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(case):
    base = Workload(name="edge", dtype=DTYPE_BF16, h_q=8, h_kv=2, head_dim=128,
                    seqlens_k=[700, 129, 64, 1, 333], seqlens_q=[700, 5, 64, 1, 1], block=16,
                    pool=POOL_MEAN, topk=6, n_init=16, window=32, seed=77)
    w = base.scaled(**EDGE[case])
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


DECODE_EDGE = {
    # k between the filtered search (<= 64) and the part size (128)
    "k100": dict(topk=100, block=8),
    # k above the part size: every part survives whole, full search over <= 512 survivors
    "k300": dict(topk=300, block=8),
    # per-sequence k, zero for some rows
    "k_per_seq": dict(topk=7, topk_per_seq=[0, 5, 0, 7, 2]),
    # a single 128-candidate part
    "one_part": dict(block=32, topk=9),
}


# selection plans for rows of one query with at most 1024 candidates: parts of 128
# candidates + a merge (few rows), or one 16-wavefront workgroup per (row, KV head)
ROW_PLANS = {"parts": "1", "fused": "5"}


@pytest.mark.parametrize("plan", list(ROW_PLANS))
@pytest.mark.parametrize("case", list(DECODE_EDGE) + ["default", "max_cand"])
def test_decode_selection_cases(case, plan, monkeypatch):
    """One query per sequence: both selection plans for rows of up to 1024 candidates."""
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", ROW_PLANS[plan])
    w = small("bf16_decode_32k")
    if case == "max_cand":                # 1024 candidates: two scoring passes of the fused plan
        w = w.scaled(block=4, topk=40, n_init=0, window=1, seqlens_k=[4096, 4096, 3001, 1030, 130])
        assert w.nb_max == 1024
    elif case != "default":
        w = w.scaled(**DECODE_EDGE[case])
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_fp32_d64_decode_and_prefill_mix():
    w = Workload(name="mix", dtype=DTYPE_F32, h_q=4, h_kv=1, head_dim=64, seqlens_k=[300, 1200, 95],
                 seqlens_q=[300, 3, 95], block=32, pool=POOL_MEAN, topk=3, n_init=32, window=64, seed=5)
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_explicit_query_positions():
    """q_pos0 given (queries not right-aligned): selection and causality follow it."""
    w = Workload(name="qpos", dtype=DTYPE_BF16, h_q=4, h_kv=2, head_dim=128, seqlens_k=[900, 500],
                 seqlens_q=[40, 7], block=16, pool=POOL_MEAN, topk=5, n_init=16, window=48, seed=9)
    q_pos0 = [600, 100]
    x, xg = parity.gen_pair(w)
    p = sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device="cuda", h_q=4, h_kv=2, head_dim=128,
                               block=16, topk=5, n_init=16, window=48, q_pos0=q_pos0, dtype=torch.bfloat16)
    kc = sa.compress(p, xg["k"])
    idx, n_idx = sa.select(p, xg["q"], kc, xg["k"])
    out = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx)
    kco = oracle.compress(w, x["k"])
    sel = oracle.select(w, x["q"], kco, x["k"], q_pos0=q_pos0)
    gi, gn = idx.cpu().numpy(), n_idx.cpu().numpy()
    for r, (row, c) in enumerate(zip(sel["rows"], sel["heads"])):
        assert gn[c, row] == sel["n"][r]
        assert list(gi[c, row, :gn[c, row]]) == list(sel["idx"][r, :sel["n"][r]]) or parity.near_tie(sel, r)
    att = oracle.attend(w, x["q"], x["k"], x["v"], gi, gn, q_pos0=q_pos0)
    parity.check_output(w, out.float().cpu().reshape(-1, 128), att["out"])


def test_shared_selection_drafts_share_one_set():
    w = small("bf16_draft_decode")
    x, xg = parity.gen_pair(w)
    r = parity.full_check(w, x, xg)
    assert r["gpu"]["idx"].shape[1] == w.batch      # one row per sequence


def test_split_selection_path():
    """Shared token-level rows with more candidates than the fused kernel holds in LDS:
    split scoring into the workspace + workgroup radix top-k."""
    from workloads import draft_decode
    w = draft_decode(batch=3, median=5000, lo=4500, hi=9000, seed=4321)
    assert w.max_k > 4096
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def _integer_inputs(w, lo=-2, hi=2, seed=0):
    """Small-integer Q and K: every score is exact in fp32 and fp64, so ties are exact
    and the GPU must resolve them exactly like the oracle (lower index first)."""
    g = torch.Generator().manual_seed(seed)
    x = generate(w)
    x["q"] = torch.randint(lo, hi + 1, x["q"].shape, generator=g).to(x["q"].dtype)
    x["k"] = torch.randint(lo, hi + 1, x["k"].shape, generator=g).to(x["k"].dtype)
    return x


@pytest.mark.parametrize("case", ["wave", "compact", "tile", "tile_long"])
def test_topk_exact_ties(case):
    from workloads import draft_decode
    if case == "compact":      # token-level shared rows with > 2048 candidates
        w = draft_decode(batch=3, median=5000, lo=4500, hi=9000, seed=11)
    elif case == "wave":       # decode rows, <= 2048 candidates
        w = small("bf16_decode_32k")
    elif case == "tile":       # prefill rows (MFMA fp32 scores) with 4097 candidates, mean pooling
        w = small("bf16_chunked_prefill_1m").scaled(pool=POOL_MEAN)
    else:                      # rows long enough for the top-k to start from the group maxima
        w = small("bf16_chunked_prefill_1m").scaled(pool=POOL_MEAN, seqlens_k=[65536 + 3], seqlens_q=[64])
    x = _integer_inputs(w)
    parity.full_check(w, x, parity.to_device(x))


@pytest.mark.parametrize("n_k,n_q,k", [(65536 + 3, 96, 64), (270000 + 1, 40, 512), (131072 + 17, 33, 200)])
def test_long_rows_group_maxima(n_k, n_q, k):
    """Prefill rows of >= 4k groups of 32 candidates: the top-k reads only the groups whose
    score maximum (kept by the scoring kernel) reaches the k-th largest group maximum."""
    w = small("bf16_chunked_prefill_1m").scaled(seqlens_k=[n_k], seqlens_q=[n_q], topk=k)
    assert (n_k - n_q - w.window) // w.block - 1 >= 4 * 32 * k        # every row takes that path
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_long_rows_per_thread_maxima():
    """Rows of >= 65536 candidates scored per head (the max-over-heads group score, no
    group maxima): the top-k gathers the keys above the k-th largest per-thread maximum."""
    from workloads import SELECT_MAX
    w = small("bf16_chunked_prefill_1m").scaled(seqlens_k=[270000 + 1], seqlens_q=[24], topk=512,
                                                select_mode=SELECT_MAX)
    assert (w.seqlens_k[0] - 24 - w.window) // w.block - 1 >= 65536
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_topk_all_scores_equal():
    """Every candidate scores the same: the k lowest indices (all-equal keys overflow the
    compaction buffer of the large-row top-k)."""
    from workloads import draft_decode
    w = draft_decode(batch=2, median=9000, lo=8000, hi=12000, seed=12)
    x = generate(w)
    x["k"] = torch.ones_like(x["k"])
    parity.full_check(w, x, parity.to_device(x))


def test_deterministic():
    w = small("bf16_prefill_128k")
    x, xg = parity.gen_pair(w)
    a = parity.run_gpu(w, xg)
    b = parity.run_gpu(w, xg)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["n_idx"], b["n_idx"])
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])


def test_select_workspace_reuse():
    """Decode rows are scored in parts whose survivors go through the workspace; one
    workspace, left with stale contents, serves repeated calls."""
    w = small("bf16_decode_32k")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"])
    sel_b, _ = sa.workspace_size(p)
    assert sel_b > 0
    ws = torch.full((sel_b,), 0xAB, dtype=torch.uint8, device="cuda")
    ref = None
    for _ in range(3):
        idx = torch.full((w.h_kv, p.rows, w.topk), -7, dtype=torch.int32, device="cuda")
        n_idx = torch.full((w.h_kv, p.rows), -7, dtype=torch.int32, device="cuda")
        sa.select(p, xg["q"], kc, xg["k"], idx, n_idx, ws=ws)
        torch.cuda.synchronize()
        got = (idx.cpu().numpy(), n_idx.cpu().numpy())
        if ref is None:
            ref = got
            parity.check_select(w, x, oracle.compress(w, x["k"]), got[0], got[1])
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_compress_tail_matches_full():
    w = small("bf16_decode_32k")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    full = sa.compress(p, xg["k"])
    tail = torch.full_like(full, float("nan"))
    sa.compress_tail(p, 2, xg["k"], tail)
    for b, n in enumerate(w.seqlens_k):
        nb = -(-n // w.block)
        lo = max(0, nb - 2)
        assert torch.equal(tail[:, b, lo:nb], full[:, b, lo:nb])
        assert torch.isnan(tail[:, b, :lo]).all()


# ---------------------------------------------------------------- long tile unions

def test_prefill_long_tile_union():
    """Shared-tile prefill attention over long tile unions: iid scores over 768 blocks with
    k = 64, so a 64-query workgroup walks most of the sequence's tiles, each tile live for
    only some of its rows.  Sampled outputs and lse against the oracle on the GPU's own table."""
    w = Workload(name="long_union", dtype=DTYPE_BF16, h_q=8, h_kv=2, head_dim=128, seqlens_k=[49152],
                 seqlens_q=[512], block=64, pool=POOL_MEAN, topk=64, n_init=64, window=512, seed=31)
    x, xg = parity.gen_pair(w)
    gp = parity.run_gpu(w, xg)
    # the union a 64-query workgroup walks: selected blocks + init + window tiles
    q0 = w.seqlens_k[0] - w.seqlens_q[0]
    longest = 0
    for c in range(w.h_kv):
        for t in range(0, w.seqlens_q[0], 64):
            tiles = set()
            for r in range(t, t + 64):
                tiles.update(gp["idx"][c, r, :gp["n_idx"][c, r]].tolist())
            p_first, p_last = q0 + t, q0 + t + 63
            tiles.update(range(0, (min(w.n_init, p_last + 1) + 63) // 64))
            tiles.update(range(max(w.n_init, p_first - w.window + 1) // 64, p_last // 64 + 1))
            longest = max(longest, len(tiles))
    assert longest > 700, f"the longest union has only {longest} tiles"
    rng = np.random.default_rng(3)
    reqs = rng.choice(w.total_q, size=384, replace=False)
    hs = rng.integers(0, w.h_q, size=len(reqs))
    att = oracle.attend(w, x["q"], x["k"], x["v"], gp["idx"], gp["n_idx"], reqs=reqs, heads=hs)
    gout = gp["out"].reshape(w.total_q, w.h_q, w.head_dim)[reqs, hs].double().numpy()
    parity.check_output(w, gout, att["out"])
    lse_g = gp["lse"][torch.from_numpy(hs), torch.from_numpy(reqs)].double().numpy()
    assert np.abs(lse_g - att["lse"]).max() < parity.lse_tol(w)


# ---------------------------------------------------------------- full size, sampled

def _sampled(w, n_rows, n_req, seed=0):
    rng = np.random.default_rng(seed)
    x, xg = parity.gen_pair(w, gen_on_device=True)
    gp = parity.run_gpu(w, xg)
    kc = oracle.compress(w, x["k"]) if w.block > 1 else None
    if kc is not None:
        bsel = rng.choice(w.batch, size=min(w.batch, 4), replace=False)
        for b in bsel:
            sub = w.scaled(seqlens_k=[w.seqlens_k[b]], seqlens_q=[w.seqlens_q[b]])
            parity.check_compress(sub, gp["k_cmp"][:, b:b + 1], kc[:, b:b + 1])
    rows = rng.choice(w.rows, size=min(w.rows, n_rows), replace=False)
    rows = np.repeat(rows, w.h_kv)
    heads = np.tile(np.arange(w.h_kv), len(rows) // w.h_kv)
    sel, n_flag = parity.check_select(w, x, kc, gp["idx"], gp["n_idx"], rows=rows, heads=heads)
    reqs = rng.choice(w.total_q, size=min(w.total_q, n_req), replace=False)
    hs = rng.integers(0, w.h_q, size=len(reqs))
    att = oracle.attend(w, x["q"], x["k"], x["v"], gp["idx"], gp["n_idx"], reqs=reqs, heads=hs)
    gout = gp["out"].reshape(w.total_q, w.h_q, w.head_dim)[reqs, hs].double().numpy()
    parity.check_output(w, gout, att["out"])
    lse_g = gp["lse"][torch.from_numpy(hs), torch.from_numpy(reqs)].double().numpy()
    assert np.abs(lse_g - att["lse"]).max() < parity.lse_tol(w)
    # GPU attention on a table whose sampled rows hold the oracle's selection
    idx2, n2 = gp["idx"].copy(), gp["n_idx"].copy()
    idx2[sel["heads"], sel["rows"]] = sel["idx"]
    n2[sel["heads"], sel["rows"]] = sel["n"]
    out2 = sa.fwd(gp["p"], xg["q"], xg["k"], xg["v"], torch.from_numpy(idx2).cuda(), torch.from_numpy(n2).cuda())
    row_of = (lambda i: np.searchsorted(np.cumsum(w.seqlens_q), i, side="right")) if w.shared_selection \
        else (lambda i: i)
    mask = np.isin(np.array([row_of(i) for i in reqs]), sel["rows"])
    if mask.any():
        att2 = oracle.attend(w, x["q"], x["k"], x["v"], idx2, n2, reqs=reqs[mask], heads=hs[mask])
        g2 = out2.float().cpu().reshape(w.total_q, w.h_q, w.head_dim)[reqs[mask], hs[mask]].double().numpy()
        parity.check_output(w, g2, att2["out"], "output on oracle rows")
    return n_flag


def test_full_decode_32k_sampled():
    parity_flags = _sampled(FULL["bf16_decode_32k"](), n_rows=32, n_req=512)
    assert parity_flags <= 8


def test_full_prefill_128k_sampled():
    _sampled(FULL["bf16_prefill_128k"](), n_rows=96, n_req=4096)


def test_full_draft_decode_sampled():
    _sampled(FULL["bf16_draft_decode"](), n_rows=64, n_req=768)


def test_full_chunked_prefill_1m_sampled():
    _sampled(FULL["bf16_chunked_prefill_1m"](), n_rows=24, n_req=2048)


# ---------------------------------------------------------------- full size, every row

def _every_row(name):
    w = FULL[name]()
    x, xg = parity.gen_pair(w, gen_on_device=True)
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"])
    idx, n_idx = sa.select(p, xg["q"], kc, xg["k"])
    torch.cuda.synchronize()
    n_diff = parity.check_select_every_row(w, x, oracle.compress(w, x["k"]), idx.cpu().numpy(),
                                           n_idx.cpu().numpy())
    print(f"{name}: {w.rows * w.h_kv} (row, KV head) selections, {n_diff} near ties that differ")
    return n_diff


def test_full_prefill_128k_every_row():
    """Every one of the 131072 x 8 selections of the 128K prefill against the oracle."""
    _every_row("bf16_prefill_128k")


def test_full_chunked_prefill_1m_every_row():
    """Every one of the 4096 selections (262144 candidate groups each) of the 1M-token chunk."""
    _every_row("bf16_chunked_prefill_1m")
