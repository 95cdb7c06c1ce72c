"""A decode step's append and selection in one call (sparse_attn_append_select),
through the C ABI (needs an MI355X).

The reference is the two calls it replaces: sparse_attn_append_kv, then
sparse_attn_select on the grown cache.  Both start from a cache whose new rows are
NaN and from pooled keys whose touched blocks are NaN, so a selection that read a
block the same launch re-pools, or an append that missed a row, shows up.  The cache,
the pooled keys and the selection table must equal the reference bit for bit: the
append's work items are the append kernel's and the selection reads the same keys.
Decode rows take the one-launch path (forced at small sizes with the row-plan
override); shared draft rows, and decode rows under the part plan, take two launches.
"""
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import FULL, POOL_L2SUM, generate, page_layout, small, to_pages, token_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _params(w, layout):
    p = parity.params_for(w)
    if layout is None:
        return p
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device="cuda", h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk, n_init=w.n_init,
                                  window=w.window, shared_selection=w.shared_selection, topk_per_seq=w.topk_per_seq,
                                  dtype=p.dtype, pool_overlap=w.pool_overlap,
                                  block_table=layout.block_table.cuda(), page_size=layout.page_size)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _compare(w, xg, layout=None):
    p = _params(w, layout)
    new, k_off = [], 0                               # packed rows of the new tokens
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        new.extend(range(k_off + nk - nq, k_off + nk))
        k_off += nk
    new = torch.tensor(new, device="cuda")
    k_new, v_new = xg["k"][new].contiguous(), xg["v"][new].contiguous()
    k_full = xg["k"] if layout is None else to_pages(xg["k"], layout)
    v_full = xg["v"] if layout is None else to_pages(xg["v"], layout)
    slots = new if layout is None else token_rows(layout).cuda()[new]
    kc = sa.compress(p, k_full) if w.block > 1 else None
    if kc is not None:          # the blocks the append re-pools start out NaN
        for b, (nk, nq) in enumerate(zip(w.seqlens_k, w.seqlens_q)):
            lo = (nk - nq) // w.block
            hi = min((nk + w.block - 1) // w.block, (nk - 1 + w.pool_overlap) // w.block + 1)
            kc[:, b, lo:hi] = float("nan")

    def stale():
        k, v = k_full.clone(), v_full.clone()
        k[slots], v[slots] = float("nan"), float("nan")
        return k, v, (kc.clone() if kc is not None else None)

    k1, v1, kc1 = stale()
    sa.append_kv(p, k_new, v_new, k1, v1, kc1)
    idx1, n1 = sa.select(p, xg["q"], kc1, k1)
    k2, v2, kc2 = stale()
    idx2, n2 = sa.append_select(p, k_new, v_new, k2, v2, kc2, xg["q"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(k1), _bits(k2)) and torch.equal(_bits(v1), _bits(v2))
    assert torch.equal(k2[slots], k_new) and torch.equal(v2[slots], v_new)
    if kc is not None:
        assert torch.equal(_bits(kc1), _bits(kc2))
    assert torch.equal(idx1, idx2) and torch.equal(n1, n2)
    return idx2, n2


CASES = {
    "decode": lambda: small("bf16_decode_32k"),
    "decode_overlap": lambda: small("bf16_decode_32k").scaled(pool_overlap=40),
    "decode_l2sum_g4": lambda: small("bf16_decode_32k").scaled(pool=POOL_L2SUM, block=4, topk=40, window=16),
}


@pytest.mark.parametrize("page_size", [0, 16])
@pytest.mark.parametrize("plan", ["5", "1"])           # one launch; two launches (part plan)
@pytest.mark.parametrize("case", list(CASES))
def test_append_select_matches_append_then_select(case, plan, page_size, monkeypatch):
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", plan)
    w = CASES[case]()
    x, xg = parity.gen_pair(w)
    layout = page_layout(w.seqlens_k, page_size, w.seed + 7) if page_size else None
    idx, n_idx = _compare(w, xg, layout)
    if layout is None and plan == "5":             # and the selection is the oracle's
        parity.check_select(w, x, oracle.compress(w, x["k"]), idx.cpu().numpy(), n_idx.cpu().numpy())


def test_append_select_shared_drafts_two_launches():
    w = small("bf16_draft_decode")
    x, xg = parity.gen_pair(w)
    _compare(w, xg)


def test_append_select_full_decode_32k():
    """The decode benchmark's shape: one launch by default (256 rows x KV heads)."""
    w = FULL["bf16_decode_32k"]()
    xg = generate(w, device="cuda")
    _compare(w, xg)
