"""Paged K/V caches and the decode-time append, through the C ABI (needs an MI355X).

A paged run gets the packed run's keys and values scattered over a pool by a
seeded page permutation (every pool slot that holds no token is NaN, so a read
of a wrong row poisons the result).  It must match the oracle, which reads the
packed tensors, to the bars of the packed path, and give pooled keys, tables,
outputs and lse bit-identical to the packed GPU run: the layout changes only
where a row is read from, never the arithmetic.

The append test starts from a cache whose newest rows are stale, appends them,
and checks the cache byte for byte (new rows written, no other row or pool slot
touched) and the re-pooled keys against the oracle's pooling of the grown cache.
The decode loop grows every sequence token by token (append, select, attend)
and compares each step with the oracle on that step's prefix.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import DTYPE_BF16, FULL, generate, page_layout, small, to_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _dt(w):
    return torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32


def paged_params(w, layout, seqlens_k=None, seqlens_q=None, max_k=None):
    p = sa.Params.from_lengths(seqlens_q or w.seqlens_q, seqlens_k or w.seqlens_k, device="cuda", h_q=w.h_q,
                               h_kv=w.h_kv, head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk,
                               n_init=w.n_init, window=w.window, shared_selection=w.shared_selection,
                               topk_per_seq=w.topk_per_seq, dtype=_dt(w), pool_overlap=w.pool_overlap,
                               select_mode=w.select_mode, select_tau=w.select_tau,
                               block_table=None if layout is None else layout.block_table.cuda(),
                               page_size=0 if layout is None else layout.page_size)
    if max_k is not None:
        p.s.max_k = max_k
    return p


def _valid_rows(w, kc):
    """Pooled rows j < ceil(N_b / g) of every sequence (the rows compress writes)."""
    return [kc[:, b, :-(-n // w.block)] for b, n in enumerate(w.seqlens_k)]


@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("name", list(FULL))
def test_paged_small_workloads(name, page_size):
    w = small(name)
    x, xg = parity.gen_pair(w)
    layout = page_layout(w.seqlens_k, page_size, w.seed)
    p = paged_params(w, layout)
    kp, vp = to_pages(xg["k"], layout), to_pages(xg["v"], layout)
    kc = sa.compress(p, kp) if w.block > 1 else None
    idx, n_idx = sa.select(p, xg["q"], kc, kp)
    out, lse = sa.fwd(p, xg["q"], kp, vp, idx, n_idx, want_lse=True)
    torch.cuda.synchronize()
    ref = parity.run_gpu(w, xg)
    # bit-identical to the packed run
    if kc is not None:
        for a, b in zip(_valid_rows(w, kc.cpu()), _valid_rows(w, ref["k_cmp"])):
            assert torch.equal(a, b)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"]) and np.array_equal(n_idx.cpu().numpy(), ref["n_idx"])
    assert torch.equal(out.float().cpu(), ref["out"]) and torch.equal(lse.cpu(), ref["lse"])
    # and the oracle on the packed tensors
    kc_o = oracle.compress(w, x["k"]) if w.block > 1 else None
    if kc_o is not None:
        parity.check_compress(w, kc.cpu(), kc_o)
    parity.check_select(w, x, kc_o, idx.cpu().numpy(), n_idx.cpu().numpy())
    att = oracle.attend(w, x["q"], x["k"], x["v"], idx.cpu().numpy(), n_idx.cpu().numpy())
    parity.check_output(w, out.float().cpu().reshape(-1, w.head_dim), att["out"])
    lse_g = lse.cpu().t().reshape(-1).double().numpy()
    assert np.abs(lse_g - att["lse"]).max() < parity.lse_tol(w)


def _new_rows(w):
    """Packed K/V row of every new token (query row i sits at position q0_b + i - q_off_b)."""
    rows, k_off = [], 0
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        rows.extend(range(k_off + nk - nq, k_off + nk))
        k_off += nk
    return torch.tensor(rows, dtype=torch.long)


APPEND = [("bf16_decode_32k", 0), ("bf16_decode_32k", 16), ("bf16_chunked_prefill_1m", 64),
          ("bf16_draft_decode", 1), ("bf16_prefill_128k", 32), ("tiny_fp32_prefill", 0)]


@pytest.mark.parametrize("name,page_size", APPEND)
def test_append_kv(name, page_size):
    w = small(name)
    x, xg = parity.gen_pair(w)
    new = _new_rows(w).cuda()
    k_new, v_new = xg["k"][new].contiguous(), xg["v"][new].contiguous()
    stale_k, stale_v = xg["k"].clone(), xg["v"].clone()
    stale_k[new] = 3.0                       # the rows the append will replace
    stale_v[new] = -3.0
    layout = page_layout(w.seqlens_k, page_size, w.seed + 1) if page_size else None
    p = paged_params(w, layout)
    kc_ = to_pages(stale_k, layout) if layout else stale_k
    vc_ = to_pages(stale_v, layout) if layout else stale_v
    kc = sa.compress(p, kc_) if w.block > 1 else None
    kc_before = None if kc is None else kc.clone()
    sa.append_kv(p, k_new, v_new, kc_, vc_, kc)
    torch.cuda.synchronize()
    want_k = to_pages(xg["k"], layout) if layout else xg["k"]
    want_v = to_pages(xg["v"], layout) if layout else xg["v"]
    # every row equal, NaN pool slots still NaN (equal_nan compares the poisoned slots)
    assert torch.equal(torch.isnan(kc_.float()), torch.isnan(want_k.float()))
    assert torch.equal(torch.nan_to_num(kc_.float()), torch.nan_to_num(want_k.float()))
    assert torch.equal(torch.nan_to_num(vc_.float()), torch.nan_to_num(want_v.float()))
    if kc is None:
        return
    ora = oracle.compress(w, x["k"])
    parity.check_compress(w, kc.cpu(), ora)
    # blocks without a new token are not rewritten
    for b, (nk, nq) in enumerate(zip(w.seqlens_k, w.seqlens_q)):
        j0 = (nk - nq) // w.block
        assert torch.equal(kc[:, b, :j0], kc_before[:, b, :j0])


@pytest.mark.parametrize("page_size", [16, 64])
def test_decode_loop(page_size):
    """A paged cache grows by one token per sequence and step: append (which re-pools
    the token's block), select, attend; every step equals the oracle on that step's
    prefix.  One block table and one pooled-key table, sized for the final lengths,
    serve every step."""
    steps = 5
    base = small("bf16_decode_32k")
    w = base.scaled(seqlens_q=[steps] * base.batch)        # query s of sequence b sits at N_b - steps + s
    x, xg = parity.gen_pair(w)
    final = list(w.seqlens_k)
    start = [int(v) for v in np.cumsum([0] + final[:-1])]
    layout = page_layout(final, page_size, w.seed + 2)
    t0 = [n - steps for n in final]
    # the cache before the loop holds the first t0_b tokens of every sequence; the rest is NaN
    keep = torch.cat([torch.arange(o, o + t) for o, t in zip(start, t0)]).cuda()
    k_cache = torch.full_like(xg["k"], float("nan"))
    v_cache = torch.full_like(xg["v"], float("nan"))
    k_cache[keep], v_cache[keep] = xg["k"][keep], xg["v"][keep]
    k_cache, v_cache = to_pages(k_cache, layout), to_pages(v_cache, layout)
    cap = max(final)
    p0 = paged_params(w, layout, seqlens_k=t0, seqlens_q=[1] * w.batch, max_k=cap)
    kc = torch.empty((w.h_kv, w.batch, p0.nb_max, w.head_dim), dtype=torch.float32, device="cuda")
    sa.compress(p0, k_cache, kc)
    for s in range(steps):
        lens = [t + s + 1 for t in t0]
        rows = torch.tensor([b * steps + s for b in range(w.batch)])
        new = torch.tensor([start[b] + lens[b] - 1 for b in range(w.batch)]).cuda()
        p = paged_params(w, layout, seqlens_k=lens, seqlens_q=[1] * w.batch, max_k=cap)
        q = xg["q"][rows.cuda()].contiguous()
        sa.append_kv(p, xg["k"][new].contiguous(), xg["v"][new].contiguous(), k_cache, v_cache, kc)
        idx, n_idx = sa.select(p, q, kc, k_cache)
        out, lse = sa.fwd(p, q, k_cache, v_cache, idx, n_idx, want_lse=True)
        torch.cuda.synchronize()
        # the oracle on this step's prefix
        ws = w.scaled(seqlens_k=lens, seqlens_q=[1] * w.batch)
        pre = torch.cat([torch.arange(start[b], start[b] + lens[b]) for b in range(w.batch)])
        xs = {"q": x["q"][rows].contiguous(), "k": x["k"][pre].contiguous(), "v": x["v"][pre].contiguous()}
        kc_o = oracle.compress(ws, xs["k"])
        got = kc.cpu()
        for b, n in enumerate(lens):
            nb = -(-n // w.block)
            diff = (got[:, b, :nb].double().numpy() - kc_o[:, b, :nb])
            tol = 2e-6 * np.maximum(1.0, np.abs(kc_o[:, b, :nb]).max(axis=-1, keepdims=True))
            assert (np.abs(diff) <= tol).all(), f"step {s}: pooled keys of sequence {b}"
        parity.check_select(ws, xs, kc_o, idx.cpu().numpy(), n_idx.cpu().numpy())
        att = oracle.attend(ws, xs["q"], xs["k"], xs["v"], idx.cpu().numpy(), n_idx.cpu().numpy())
        parity.check_output(ws, out.float().cpu().reshape(-1, w.head_dim), att["out"], f"step {s}")
        lse_g = lse.cpu().t().reshape(-1).double().numpy()
        assert np.abs(lse_g - att["lse"]).max() < parity.lse_tol(ws)


def test_full_decode_32k_paged_sampled():
    """The benchmark's decode step on a 64-token-page cache: sampled rows and requests
    against the oracle, and the whole output equal to the packed run's."""
    w = FULL["bf16_decode_32k"]()
    xg = generate(w, device="cuda")
    layout = page_layout(w.seqlens_k, 64, w.seed)
    p = paged_params(w, layout)
    kp, vp = to_pages(xg["k"], layout), to_pages(xg["v"], layout)
    kc = sa.compress(p, kp)
    idx, n_idx = sa.select(p, xg["q"], kc, kp)
    out = sa.fwd(p, xg["q"], kp, vp, idx, n_idx)
    ref = parity.run_gpu(w, xg)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"]) and np.array_equal(n_idx.cpu().numpy(), ref["n_idx"])
    assert torch.equal(out.float().cpu(), ref["out"])
    del kp, vp
    rng = np.random.default_rng(3)
    x = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in xg.items()}
    kc_o = oracle.compress(w, x["k"])
    rows = np.repeat(rng.choice(w.rows, size=8, replace=False), w.h_kv)
    heads = np.tile(np.arange(w.h_kv), len(rows) // w.h_kv)
    parity.check_select(w, x, kc_o, idx.cpu().numpy(), n_idx.cpu().numpy(), rows=rows, heads=heads)
    reqs = rng.choice(w.total_q, size=32, replace=False)
    hs = rng.integers(0, w.h_q, size=len(reqs))
    att = oracle.attend(w, x["q"], x["k"], x["v"], idx.cpu().numpy(), n_idx.cpu().numpy(), reqs=reqs, heads=hs)
    gout = out.float().cpu().reshape(w.total_q, w.h_q, w.head_dim)[reqs, hs].double().numpy()
    parity.check_output(w, gout, att["out"])
