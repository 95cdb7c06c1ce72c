"""Selector variants through the C ABI against the oracle (needs an MI355X):
overlapping pooling windows (kernel g + o, stride g), the group score as the sum
of per-head softmaxes over the candidates, the group score as the max over
heads, and the S3R refresh: selection by the attention mass of a dense verify
pass (whose lse the GPU's own dense sparse_attn_fwd provides; the oracle
computes its own).  Every stage is compared to the bars of the default path (pooled keys,
index sets with the near-tie rule on the mode's own scores, outputs)."""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import FULL, SELECT_ATTN, SELECT_MAX, SELECT_SOFTMAX, SELECT_SUM, generate, page_layout, small, to_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


MODES = {"max": dict(select_mode=SELECT_MAX), "softmax": dict(select_mode=SELECT_SOFTMAX),
         "softmax_tau": dict(select_mode=SELECT_SOFTMAX, select_tau=0.7)}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(FULL))
def test_group_score_modes(name, mode):
    w = small(name).scaled(**MODES[mode])
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


OVERLAP = [("bf16_decode_32k", 16), ("bf16_decode_32k", 63), ("bf16_prefill_128k", 40),
           ("bf16_chunked_prefill_1m", 2), ("tiny_fp32_prefill", 32)]


@pytest.mark.parametrize("name,o", OVERLAP)
def test_overlapping_pooling(name, o):
    w = small(name).scaled(pool_overlap=o)
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


def test_overlap_with_max_heads():
    w = small("bf16_decode_32k").scaled(pool_overlap=32, select_mode=SELECT_MAX, topk=11)
    x, xg = parity.gen_pair(w)
    parity.full_check(w, x, xg)


@pytest.mark.parametrize("o", [5, 64, 130])
def test_append_with_overlap(o):
    """Appending re-pools every block whose window holds a new token (the new tokens'
    own blocks and the blocks up to o tokens after them)."""
    w = small("bf16_prefill_128k").scaled(seqlens_k=[1500, 900], seqlens_q=[70, 9], pool_overlap=o)
    x, xg = parity.gen_pair(w)
    rows, k_off = [], 0
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        rows.extend(range(k_off + nk - nq, k_off + nk))
        k_off += nk
    new = torch.tensor(rows, device="cuda")
    k, v = xg["k"].clone(), xg["v"].clone()
    k[new], v[new] = 5.0, -5.0
    p = parity.params_for(w)
    kc = sa.compress(p, k)
    sa.append_kv(p, xg["k"][new].contiguous(), xg["v"][new].contiguous(), k, v, kc)
    torch.cuda.synchronize()
    assert torch.equal(k, xg["k"]) and torch.equal(v, xg["v"])
    parity.check_compress(w, kc.cpu(), oracle.compress(w, x["k"]))


def _sampled_decode(w, n_rows=16, n_req=256, seed=5):
    rng = np.random.default_rng(seed)
    xg = generate(w, device="cuda")
    gp = parity.run_gpu(w, xg)
    x = {k: (t.cpu() if isinstance(t, torch.Tensor) else t) for k, t in xg.items()}
    kc = oracle.compress(w, x["k"]) if w.block > 1 else None
    rows = np.repeat(rng.choice(w.rows, size=min(w.rows, n_rows), replace=False), w.h_kv)
    heads = np.tile(np.arange(w.h_kv), len(rows) // w.h_kv)
    _, flagged = parity.check_select(w, x, kc, gp["idx"], gp["n_idx"], rows=rows, heads=heads)
    reqs = rng.choice(w.total_q, size=min(w.total_q, n_req), replace=False)
    hs = rng.integers(0, w.h_q, size=len(reqs))
    att = oracle.attend(w, x["q"], x["k"], x["v"], gp["idx"], gp["n_idx"], reqs=reqs, heads=hs)
    gout = gp["out"].reshape(w.total_q, w.h_q, w.head_dim)[reqs, hs].double().numpy()
    parity.check_output(w, gout, att["out"])
    return flagged


@pytest.mark.parametrize("mode", ["max", "softmax"])
def test_full_decode_32k_modes_sampled(mode):
    """The decode benchmark's shape with each variant group score (sampled rows)."""
    assert _sampled_decode(FULL["bf16_decode_32k"]().scaled(**MODES[mode])) <= 8


def test_full_draft_decode_max_sampled():
    _sampled_decode(FULL["bf16_draft_decode"]().scaled(select_mode=SELECT_MAX), n_rows=16, n_req=256)


def _verify_lse(w, xg, k=None, v=None, layout=None):
    """The dense verify pass on the GPU: a table keeping every candidate, attention with lse."""
    wd = w.scaled(select_mode=SELECT_SUM, topk=max(w.seqlens_k), topk_per_seq=None)
    p = parity.params_for(wd) if layout is None else _paged(wd, layout)
    k = xg["k"] if k is None else k
    v = xg["v"] if v is None else v
    kc = sa.compress(p, k) if wd.block > 1 else None
    idx, n_idx = sa.select(p, xg["q"], kc, k)
    _, lse = sa.fwd(p, xg["q"], k, v, idx, n_idx, want_lse=True)
    return lse


def _paged(w, layout):
    p = parity.params_for(w)
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device="cuda", h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk, n_init=w.n_init,
                                  window=w.window, shared_selection=w.shared_selection,
                                  topk_per_seq=w.topk_per_seq, dtype=p.dtype, select_mode=w.select_mode,
                                  block_table=layout.block_table.cuda(), page_size=layout.page_size)


@pytest.mark.parametrize("name", ["bf16_draft_decode", "bf16_decode_32k", "tiny_fp32_prefill"])
def test_attention_mass_refresh(name):
    """Every row's selection by verify attention mass equals the oracle's (near-tie rule on
    the masses).  The verify pass keeps every candidate, so it is dense (window >= g here)."""
    w = small(name).scaled(select_mode=SELECT_ATTN)
    x, xg = parity.gen_pair(w)
    lse = _verify_lse(w, xg)
    p = parity.params_for(w)
    idx, n_idx = sa.select(p, xg["q"], None, xg["k"], attn_lse=lse)
    torch.cuda.synchronize()
    parity.check_select(w, x, None, idx.cpu().numpy(), n_idx.cpu().numpy())


def test_attention_mass_refresh_vector_kernel(monkeypatch):
    """Draft rows (bf16 token keys, <= 16 (query, head) pairs) take the matrix-core scorer;
    the vector scorer, which serves every other shape, on the same rows."""
    monkeypatch.setenv("SPARSE_ATTN_ATTN_VALU", "1")
    test_attention_mass_refresh("bf16_draft_decode")


def test_attention_mass_refresh_paged():
    w = small("bf16_draft_decode").scaled(select_mode=SELECT_ATTN)
    x, xg = parity.gen_pair(w)
    layout = page_layout(w.seqlens_k, 16, w.seed + 3)
    kp, vp = to_pages(xg["k"], layout), to_pages(xg["v"], layout)
    lse = _verify_lse(w, xg, kp, vp, layout)
    idx, n_idx = sa.select(_paged(w, layout), xg["q"], None, kp, attn_lse=lse)
    torch.cuda.synchronize()
    parity.check_select(w, x, None, idx.cpu().numpy(), n_idx.cpu().numpy())


def test_full_draft_decode_refresh_sampled():
    """The S3R round at full size: dense verify of the 6 drafts of 64 sequences, then the
    refreshed selection (sampled rows against the oracle)."""
    w = FULL["bf16_draft_decode"]().scaled(select_mode=SELECT_ATTN)
    xg = generate(w, device="cuda")
    lse = _verify_lse(w, xg)
    idx, n_idx = sa.select(parity.params_for(w), xg["q"], None, xg["k"], attn_lse=lse)
    torch.cuda.synchronize()
    x = {k: (t.cpu() if isinstance(t, torch.Tensor) else t) for k, t in xg.items()}
    rng = np.random.default_rng(11)
    rows = np.repeat(rng.choice(w.rows, size=12, replace=False), w.h_kv)
    heads = np.tile(np.arange(w.h_kv), len(rows) // w.h_kv)
    parity.check_select(w, x, None, idx.cpu().numpy(), n_idx.cpu().numpy(), rows=rows, heads=heads)
