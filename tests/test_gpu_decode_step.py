"""One decode step in one call (sparse_attn_decode_step) through the C ABI (needs an
MI355X).

The reference is the three calls it replaces: sparse_attn_append_kv, then
sparse_attn_select and sparse_attn_fwd on the grown cache.  Both start from a cache
whose new rows are NaN and from pooled keys whose touched blocks are NaN.  The
cache, the pooled keys and the selection table must equal the reference bit for
bit (the append and the selection are the row plan's own code); the output and lse
must agree with sparse_attn_fwd's to fp32 rounding (the attention's wavefronts merge
in another order) and meet the oracle's bars on the GPU's table.  Decode batches
take the one-launch path (forced at small sizes with the row-plan override); under
the part plan the call runs the three launches and must match them bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import FULL, POOL_L2SUM, decode_32k, generate, page_layout, small, to_pages, token_rows

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
                                  window=w.window, dtype=p.dtype, pool_overlap=w.pool_overlap,
                                  block_table=layout.block_table.cuda(), page_size=layout.page_size)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _step(w, xg, layout=None, exact_out=False):
    p = _params(w, layout)
    new, k_off = [], 0
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        new.extend(range(k_off + nk - nq, k_off + nk))
        k_off += nk
    new = torch.tensor(new, device="cuda")
    k_new, v_new = xg["k"][new].contiguous(), xg["v"][new].contiguous()
    k_full = xg["k"] if layout is None else to_pages(xg["k"], layout)
    v_full = xg["v"] if layout is None else to_pages(xg["v"], layout)
    slots = new if layout is None else token_rows(layout).cuda()[new]
    kc = sa.compress(p, k_full)
    for b, (nk, nq) in enumerate(zip(w.seqlens_k, w.seqlens_q)):
        lo = (nk - nq) // w.block
        hi = min((nk + w.block - 1) // w.block, (nk - 1 + w.pool_overlap) // w.block + 1)
        kc[:, b, lo:hi] = float("nan")

    def stale():
        k, v = k_full.clone(), v_full.clone()
        k[slots], v[slots] = float("nan"), float("nan")
        return k, v, kc.clone()

    k1, v1, kc1 = stale()
    sa.append_kv(p, k_new, v_new, k1, v1, kc1)
    idx1, n1 = sa.select(p, xg["q"], kc1, k1)
    out1, lse1 = sa.fwd(p, xg["q"], k1, v1, idx1, n1, want_lse=True)
    k2, v2, kc2 = stale()
    out2, lse2, idx2, n2 = sa.decode_step(p, k_new, v_new, k2, v2, kc2, xg["q"], want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(k1), _bits(k2)) and torch.equal(_bits(v1), _bits(v2))
    assert torch.equal(_bits(kc1), _bits(kc2))
    assert torch.equal(idx1, idx2) and torch.equal(n1, n2)
    if exact_out:
        assert torch.equal(_bits(out1), _bits(out2)) and torch.equal(lse1, lse2)
    else:
        d = (out1.float() - out2.float()).abs().max().item()
        assert d <= 1e-2 * out1.float().abs().max().item(), d
        assert (lse1 - lse2).abs().max().item() < 1e-4
    return out2, lse2, idx2, n2


def _against_oracle(w, x, out, lse, idx, n_idx, reqs=None, heads=None):
    gi, gn = idx.cpu().numpy(), n_idx.cpu().numpy()
    att = oracle.attend(w, x["q"], x["k"], x["v"], gi, gn, reqs=reqs, heads=heads)
    o = out.float().cpu().reshape(w.total_q, w.h_q, w.head_dim)
    lg = lse.cpu()
    if reqs is None:
        parity.check_output(w, o.reshape(-1, w.head_dim), att["out"])
        lse_g = lg.t().reshape(-1).double().numpy()
    else:
        parity.check_output(w, o[reqs, heads].double().numpy(), att["out"])
        lse_g = lg[torch.from_numpy(heads), torch.from_numpy(reqs)].double().numpy()
    assert np.abs(lse_g - att["lse"]).max() < parity.lse_tol(w)


def _ragged32():
    lens = [700 + (977 * i) % 3500 for i in range(32)]
    return decode_32k().scaled(seqlens_k=lens, seqlens_q=[1] * 32, name="bf16_decode_ragged32")


CASES = {
    "ragged32": _ragged32,                               # 256 rows x KV heads: one launch by default
    "small": lambda: small("bf16_decode_32k"),
    "overlap": lambda: small("bf16_decode_32k").scaled(pool_overlap=40),
    "l2sum_g4": lambda: small("bf16_decode_32k").scaled(pool=POOL_L2SUM, block=4, topk=40, window=16),
    "g8_d64": lambda: small("bf16_decode_32k").scaled(h_q=64, h_kv=8, head_dim=64),
    "k_covers_all": lambda: small("bf16_decode_32k").scaled(topk=100),
}


@pytest.mark.parametrize("page_size", [0, 16])
@pytest.mark.parametrize("case", list(CASES))
def test_decode_step_one_launch(case, page_size, monkeypatch):
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", "5")
    w = CASES[case]()
    x, xg = parity.gen_pair(w)
    layout = page_layout(w.seqlens_k, page_size, w.seed + 7) if page_size else None
    out, lse, idx, n_idx = _step(w, xg, layout)
    if layout is None:
        parity.check_select(w, x, oracle.compress(w, x["k"]), idx.cpu().numpy(), n_idx.cpu().numpy())
        _against_oracle(w, x, out, lse, idx, n_idx)


def test_decode_step_three_launches_match_exactly(monkeypatch):
    """Under the part plan the step runs the three launches: bit-identical to them."""
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", "1")
    w = small("bf16_decode_32k")
    _, xg = parity.gen_pair(w)
    _step(w, xg, exact_out=True)


def test_decode_step_full_decode_32k():
    """The decode benchmark's shape (one launch), against the three calls and, on sampled
    (query, head) pairs, the oracle."""
    w = FULL["bf16_decode_32k"]()
    x, xg = parity.gen_pair(w, gen_on_device=True)
    out, lse, idx, n_idx = _step(w, xg)
    rows = np.arange(w.rows)
    parity.check_select(w, x, oracle.compress(w, x["k"]), idx.cpu().numpy(), n_idx.cpu().numpy(),
                        rows=np.repeat(rows, w.h_kv), heads=np.tile(np.arange(w.h_kv), w.rows))
    rng = np.random.default_rng(3)
    reqs = rng.integers(0, w.total_q, size=256)
    heads = rng.integers(0, w.h_q, size=256)
    _against_oracle(w, x, out, lse, idx, n_idx, reqs=reqs, heads=heads)
