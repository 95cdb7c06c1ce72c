"""Library calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The entry points launch only kernels on the caller's stream (no memsets, copies or
synchronisation), so a caller may capture them.  Each case runs the calls eagerly,
captures the same calls on the same buffers, and replays the graph several times with
eager work and synchronisations between the replays (the outputs poisoned each time);
every replay must equal the eager result bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import parity
import top_block_sparse_mean_amd as sa
from workloads import small

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _new_rows(w, k, v):
    """The last M_b tokens of every sequence: the rows a decode step or draft round appends."""
    rows, o = [], 0
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        rows.extend(range(o + nk - nq, o + nk))
        o += nk
    r = torch.tensor(rows, device=k.device)
    return k[r].contiguous(), v[r].contiguous()


def _replay_and_compare(run, outputs, poison):
    """Eager reference, then capture `run` and replay it REPLAYS times."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up off the capture stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(REPLAYS):
        poison()
        scratch.mul_(1.0001).add_(float(i))           # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert torch.equal(got, want), f"replay {i} differs from the eager calls"
    del g


def test_graph_decode_step():
    """One decode step (append, select and attend in one launch)."""
    w = small("bf16_decode_32k")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    k_new, v_new = _new_rows(w, xg["k"], xg["v"])
    k_cmp = sa.compress(p, xg["k"])
    idx = torch.empty((w.h_kv, p.rows, w.topk), dtype=torch.int32, device="cuda")
    n_idx = torch.empty((w.h_kv, p.rows), dtype=torch.int32, device="cuda")
    out = torch.empty_like(xg["q"])
    sel_b, fwd_b = sa.workspace_size(p)
    ws = torch.empty(max(sel_b, fwd_b, 16), dtype=torch.uint8, device="cuda")

    def run():
        sa.decode_step(p, k_new, v_new, xg["k"], xg["v"], k_cmp, xg["q"], idx, n_idx, out=out, ws=ws)

    def poison():
        out.fill_(float("nan"))
        idx.fill_(-7)
        n_idx.fill_(-7)

    _replay_and_compare(run, [out, idx, n_idx], poison)


def test_graph_draft_round():
    """A draft round: the drafts appended inside the selection launch, then attention."""
    w = small("bf16_draft_decode")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    k_new, v_new = _new_rows(w, xg["k"], xg["v"])
    idx = torch.empty((w.h_kv, p.rows, max(w.topk, 1)), dtype=torch.int32, device="cuda")
    n_idx = torch.empty((w.h_kv, p.rows), dtype=torch.int32, device="cuda")
    out = torch.empty_like(xg["q"])
    sel_b, fwd_b = sa.workspace_size(p)
    ws_sel = torch.empty(max(sel_b, 16), dtype=torch.uint8, device="cuda")
    ws_fwd = torch.empty(max(fwd_b, 16), dtype=torch.uint8, device="cuda")

    def run():
        sa.append_select(p, k_new, v_new, xg["k"], xg["v"], None, xg["q"], idx, n_idx, ws=ws_sel)
        sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx, out=out, ws=ws_fwd)

    def poison():
        out.fill_(float("nan"))
        idx.fill_(-7)

    _replay_and_compare(run, [out, idx, n_idx], poison)


@pytest.mark.parametrize("name", ["bf16_prefill_128k", "bf16_chunked_prefill_1m"])
def test_graph_prefill(name):
    """A prefill pass: pooling, selection (score tiles + workspace top-k) and attention."""
    w = small(name)
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    k_cmp = torch.empty((w.h_kv, w.batch, p.nb_max, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.h_kv, p.rows, max(w.topk, 1)), dtype=torch.int32, device="cuda")
    n_idx = torch.empty((w.h_kv, p.rows), dtype=torch.int32, device="cuda")
    out = torch.empty_like(xg["q"])
    lse = torch.empty((w.h_q, w.total_q), dtype=torch.float32, device="cuda")
    sel_b, fwd_b = sa.workspace_size(p)
    ws_sel = torch.empty(max(sel_b, 16), dtype=torch.uint8, device="cuda")
    ws_fwd = torch.empty(max(fwd_b, 16), dtype=torch.uint8, device="cuda")

    def run():
        sa.compress(p, xg["k"], k_cmp)
        sa.select(p, xg["q"], k_cmp, xg["k"], idx, n_idx, ws=ws_sel)
        sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx, out=out, lse=lse, ws=ws_fwd)

    def poison():
        k_cmp.fill_(float("nan"))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        idx.fill_(-7)

    _replay_and_compare(run, [k_cmp, idx, n_idx, out, lse], poison)


def test_graph_fwd_noalloc():
    """The no-allocation attention (split partials in the library's fixed scratch)."""
    w = small("bf16_decode_32k")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    k_cmp = sa.compress(p, xg["k"])
    idx, n_idx = sa.select(p, xg["q"], k_cmp, xg["k"])
    out = torch.empty_like(xg["q"])
    lse = torch.empty((w.h_q, w.total_q), dtype=torch.float32, device="cuda")

    def run():
        sa.fwd_noalloc(p, xg["q"], xg["k"], xg["v"], idx, n_idx, out, lse)

    def poison():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    _replay_and_compare(run, [out, lse], poison)
    # and the replayed result is the allocating call's
    assert torch.equal(out, sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx))
    assert np.isfinite(lse.cpu().numpy()).all()
