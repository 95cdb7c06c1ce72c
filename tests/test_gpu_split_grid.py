"""The split scorer's packed grid against its rows x chunks grid (needs an MI355X).

With one row per sequence and a packed cache, the split plan launches only the rows'
actual chunks and each workgroup finds its (row, chunk) by a prefix sum of the rows'
chunk counts; SPARSE_ATTN_SPLIT_GRID forces the rows x (chunks of the longest row)
grid.  Both must give the same selection and boundary scores bit for bit, on lengths
that mix rows keeping every candidate (no chunk), one-chunk rows and long rows, and on
the full draft round; the mixed case is also held against the oracle.
"""
import pytest
import torch

import parity
import top_block_sparse_mean_amd as sa
from workloads import draft_decode, draft_keep

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _mixed():
    # 40 sequences: some shorter than the 256 tokens a draft keeps (every candidate kept),
    # several single-chunk rows, rows ending just past a chunk edge and a few long ones
    hist = [100, 250, 300, 511, 512, 513, 1024, 1025, 1536, 4000, 9000, 20000, 32768] + \
        [300 + (7919 * i) % 6000 for i in range(27)]
    w = draft_decode(batch=len(hist))
    keep = [draft_keep(t) for t in hist]
    topk = [max(kp - w.window, 0) for kp in keep]
    return w.scaled(seqlens_k=[t + 6 for t in hist], seqlens_q=[6] * len(hist), topk=max(topk),
                    topk_per_seq=topk, name="bf16_draft_mixed")


def _both(w, xg, monkeypatch):
    p = parity.params_for(w)
    monkeypatch.setenv("SPARSE_ATTN_SELECT_PLAN", "2")
    monkeypatch.delenv("SPARSE_ATTN_SPLIT_GRID", raising=False)
    a = sa.select(p, xg["q"], None, xg["k"], want_boundary=True)
    monkeypatch.setenv("SPARSE_ATTN_SPLIT_GRID", "1")
    b = sa.select(p, xg["q"], None, xg["k"], want_boundary=True)
    torch.cuda.synchronize()
    return a, b


def _same(a, b):
    (ia, na, ba), (ib, nb, bb) = a, b
    assert torch.equal(na, nb)
    assert torch.equal(ia, ib)
    assert torch.equal(torch.nan_to_num(ba, nan=-7.0), torch.nan_to_num(bb, nan=-7.0))


def test_packed_grid_mixed_lengths(monkeypatch):
    w = _mixed()
    x, xg = parity.gen_pair(w)
    a, b = _both(w, xg, monkeypatch)
    _same(a, b)
    parity.check_select(w, x, None, a[0].cpu().numpy(), a[1].cpu().numpy())


def test_packed_grid_full_draft_round(monkeypatch):
    w = draft_decode()
    _, xg = parity.gen_pair(w, gen_on_device=True)
    a, b = _both(w, xg, monkeypatch)
    _same(a, b)
