"""Scenarios for the library built with contract checks (run by test_gpu_contract_checks.py
in a child process whose SPARSE_ATTN_LIB names libsparse_attn_checked.so).

Valid calls on every workload's small shape (packed and paged, the full pass, the
one-launch decode step and the append) must set no check bit and still meet the oracle's
bars (the full passes); then three contract
violations that the kernels clamp are planted one at a time in a decode table -- a
selection entry far outside its row's candidate blocks, a selection count above topk,
a negative page id -- and each must set its bit while the output stays finite.
Prints one line per scenario (`name flags`) and ends with `done`.
"""
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import parity  # noqa: E402
import top_block_sparse_mean_amd as sa  # noqa: E402
from workloads import FULL, page_layout, small, to_pages  # noqa: E402


def report(name):
    torch.cuda.synchronize()
    print(name, sa.check_flags(clear=True), flush=True)


def paged_params(w, layout):
    p = parity.params_for(w)
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device="cuda", h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk, n_init=w.n_init,
                                  window=w.window, dtype=p.dtype, pool_overlap=w.pool_overlap,
                                  block_table=layout.block_table.cuda(), page_size=layout.page_size)


def main():
    assert sa.LIB_PATH.endswith("libsparse_attn_checked.so"), sa.LIB_PATH
    torch.cuda.set_device(0)
    sa.check_flags(clear=True)
    for name in FULL:                                   # valid: full pass against the oracle
        w = small(name)
        x, xg = parity.gen_pair(w)
        parity.full_check(w, x, xg)
        report(f"valid_{name}")

    w = small("bf16_decode_32k")
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"])
    idx, n_idx = sa.select(p, xg["q"], kc, xg["k"])
    out = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx)
    report("valid_decode_calls")

    # valid: the one-launch decode step (forced at this size) and the append, on a cache
    # that already holds the step's tokens (they are rewritten with the same values)
    last, off = [], 0
    for nk in w.seqlens_k:
        off += nk
        last.append(off - 1)
    last = torch.tensor(last, device="cuda")
    k_new, v_new = xg["k"][last].contiguous(), xg["v"][last].contiguous()
    os.environ["SPARSE_ATTN_SELECT_PLAN"] = "5"
    out_s, _, idx_s, n_s = sa.decode_step(p, k_new, v_new, xg["k"], xg["v"], kc, xg["q"], want_lse=True)
    del os.environ["SPARSE_ATTN_SELECT_PLAN"]
    sa.append_kv(p, k_new, v_new, xg["k"], xg["v"], kc)
    torch.cuda.synchronize()
    assert torch.isfinite(out_s.float()).all()          # (a sequence shorter than sink + window selects none)
    report("valid_decode_step")

    layout = page_layout(w.seqlens_k, 16, w.seed + 7)   # valid: paged
    pp = paged_params(w, layout)
    kp, vp = to_pages(xg["k"], layout), to_pages(xg["v"], layout)
    kcp = sa.compress(pp, kp)
    idx_p, n_p = sa.select(pp, xg["q"], kcp, kp)
    out_p = sa.fwd(pp, xg["q"], kp, vp, idx_p, n_p)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx) and torch.equal(n_p, n_idx)
    report("valid_paged")

    bad = idx.clone()                                   # an entry far past the candidates
    bad[0, 0, 1] = 1 << 20
    o = sa.fwd(p, xg["q"], xg["k"], xg["v"], bad, n_idx)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    report("bad_entry")

    bad_n = n_idx.clone()                               # a count above topk
    bad_n[0, 0] = w.topk + 3
    o = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, bad_n)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    report("bad_count")

    bt = layout.block_table.clone()                     # a negative page id
    bt[0, 0] = -1
    pb = sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device="cuda", h_q=w.h_q, h_kv=w.h_kv,
                                head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk, n_init=w.n_init,
                                window=w.window, dtype=pp.dtype, pool_overlap=w.pool_overlap,
                                block_table=bt.cuda(), page_size=layout.page_size)
    o = sa.fwd(pb, xg["q"], kp, vp, idx_p, n_p)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    report("bad_page")
    del out, out_p
    print("done", flush=True)


if __name__ == "__main__":
    main()
