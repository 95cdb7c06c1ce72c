"""Helpers that run the HIP path through the binding and compare it with the
oracle (GPU tests only).

Bars (applied element by element):
  * pooled keys: |gpu - oracle| <= 2e-6 * max(1, |oracle row|_inf)   (fp32 sums);
  * index sets: identical, except rows whose k-th and (k+1)-th oracle scores
    are a near tie (relative gap < 1e-4, or absolute gap under the floor
    1e-6 * |Qs| * max|K~| / sqrt(d)); such a row passes when the GPU set has
    the right size, holds every candidate scoring above tau + delta and none
    below tau - delta, with tau the midpoint of the two scores and delta =
    max(1e-4 * max(|s_k|, |s_k+1|), floor);
  * outputs: fp32 max-abs <= 1e-5; bf16 relative l_inf (over the whole
    output) <= 1e-2.  The oracle recomputes attention on the GPU's own index
    table, so a legitimately different near-tie set does not count against
    the attention kernel; the GPU attention is also run on the oracle's table.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import top_block_sparse_mean_amd as sa
from workloads import DTYPE_BF16, generate

REL_GAP = 1e-4
F32_ABS = 1e-5
BF16_REL = 1e-2
# Log-sum-exp: fp32 arithmetic keeps it within 1e-4.  The bf16 path rounds each
# softmax weight to bf16 (relative error <= 2^-8) before the P V product and may
# normalise by the sum of the rounded weights, so |d lse| <= log(1 + 2^-8) < 4e-3.
LSE_ABS = {"f32": 1e-4, "bf16": 4e-3}


def lse_tol(w):
    return LSE_ABS["bf16" if w.dtype == DTYPE_BF16 else "f32"]


def params_for(w, device="cuda"):
    dt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device=device, h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk,
                                  n_init=w.n_init, window=w.window, shared_selection=w.shared_selection,
                                  topk_per_seq=w.topk_per_seq, dtype=dt, pool_overlap=w.pool_overlap,
                                  select_mode=w.select_mode, select_tau=w.select_tau)


def run_gpu(w, xg, p=None):
    """compress -> select -> fwd on device tensors xg; returns CPU copies."""
    p = p or params_for(w, xg["q"].device)
    kc = sa.compress(p, xg["k"]) if w.block > 1 else None
    idx, n_idx = sa.select(p, xg["q"], kc, xg["k"])
    out, lse = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx, want_lse=True)
    torch.cuda.synchronize()
    return dict(k_cmp=None if kc is None else kc.cpu(), idx=idx.cpu().numpy(), n_idx=n_idx.cpu().numpy(),
                out=out.float().cpu(), lse=lse.cpu(), p=p)


def to_device(x, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def to_host(x):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def check_compress(w, gpu_kc, ora_kc):
    g = gpu_kc.double().numpy()
    for b in range(w.batch):
        nb = -(-w.seqlens_k[b] // w.block)
        a, o = g[:, b, :nb], ora_kc[:, b, :nb]
        tol = 2e-6 * np.maximum(1.0, np.abs(o).max(axis=-1, keepdims=True))
        bad = np.abs(a - o) > tol
        assert not bad.any(), f"pooled keys differ (seq {b}): max err {np.abs(a - o).max():.3e}"


def near_tie(sel, r):
    sk, sk1, fl = sel["sk"][r], sel["sk1"][r], sel["floor"][r]
    if math.isnan(sk) or math.isnan(sk1):
        return False
    gap = abs(sk - sk1)
    return gap < REL_GAP * max(abs(sk), abs(sk1)) or gap < fl


def check_select(w, x_host, kc_ora, gpu_idx, gpu_n, rows=None, heads=None):
    """Compare GPU tables [Hkv, rows, k] with the oracle on (row, head) requests.

    Returns (oracle selection dict, number of flagged near-tie rows)."""
    sel = oracle.select(w, x_host["q"], kc_ora, x_host["k"], rows=rows, heads=heads)
    flagged, bad = [], []
    for r, (row, c) in enumerate(zip(sel["rows"], sel["heads"])):
        n = int(sel["n"][r])
        g_n = int(gpu_n[c, row])
        g_set = list(gpu_idx[c, row, :g_n]) if g_n > 0 else []
        if g_n != n:
            bad.append((row, c, "count", g_n, n))
            continue
        if any(x != -1 for x in gpu_idx[c, row, g_n:w.topk]):
            bad.append((row, c, "padding"))
            continue
        want = list(sel["idx"][r, :n])
        if g_set == want:
            continue
        if near_tie(sel, r):
            flagged.append(r)
        else:
            bad.append((row, c, "set", g_set[:8], want[:8], sel["sk"][r], sel["sk1"][r]))
    assert not bad, f"{len(bad)} selection mismatches, first: {bad[:3]}"
    if flagged:
        fr = np.array(flagged)
        sc = oracle.select(w, x_host["q"], kc_ora, x_host["k"], rows=sel["rows"][fr], heads=sel["heads"][fr],
                           want_scores=True)
        for m, r in enumerate(fr):
            row, c = sel["rows"][r], sel["heads"][r]
            s = sc["scores"][m]
            sk, sk1, fl = sel["sk"][r], sel["sk1"][r], sel["floor"][r]
            tau, delta = 0.5 * (sk + sk1), max(REL_GAP * max(abs(sk), abs(sk1)), fl)
            g_set = set(int(j) for j in gpu_idx[c, row, :gpu_n[c, row]])
            must = set(np.nonzero(s > tau + delta)[0].tolist())
            never = set(np.nonzero(s < tau - delta)[0].tolist())
            assert must <= g_set and not (g_set & never), (row, c, "near-tie rule")
            assert all(not np.isnan(s[j]) for j in g_set), (row, c, "non-candidate selected")
    return sel, len(flagged)


def check_select_every_row(w, x_host, kc_ora, gpu_idx, gpu_n):
    """check_select over every (row, KV head) of a full-size workload: the oracle selects
    every row, the tables are compared at once, and only the rows that differ go through
    the near-tie rule (with the oracle's scores of those rows).  Returns the number of
    rows that differ (each a legitimate near tie)."""
    sel = oracle.select(w, x_host["q"], kc_ora, x_host["k"])
    o_idx, o_n = oracle.table(w, sel)
    k = o_idx.shape[2]
    g_idx = gpu_idx[:, :, :k]
    same = (gpu_n == o_n) & np.all(g_idx == o_idx, axis=2)
    if k < gpu_idx.shape[2]:
        same &= np.all(gpu_idx[:, :, k:] == -1, axis=2)
    heads, rows = np.nonzero(~same)
    if len(rows):
        check_select(w, x_host, kc_ora, gpu_idx, gpu_n, rows=rows, heads=heads)
    return len(rows)


def check_output(w, gpu_out, ora_out, what="output"):
    g = gpu_out.reshape(ora_out.shape).double().numpy() if isinstance(gpu_out, torch.Tensor) else gpu_out
    err = np.abs(g - ora_out)
    if w.dtype == DTYPE_BF16:
        rel = err.max() / np.abs(ora_out).max()
        assert rel <= BF16_REL, f"{what}: relative l_inf {rel:.3e} > {BF16_REL}"
        return rel
    assert err.max() <= F32_ABS, f"{what}: max abs {err.max():.3e} > {F32_ABS}"
    return err.max()


def full_check(w, x_host, xg=None):
    """Every stage against the oracle on all rows and requests (small workloads)."""
    xg = xg or to_device(x_host)
    gp = run_gpu(w, xg)
    kc = oracle.compress(w, x_host["k"]) if w.block > 1 else None
    if kc is not None:
        check_compress(w, gp["k_cmp"], kc)
    _, n_flag = check_select(w, x_host, kc, gp["idx"], gp["n_idx"])
    # attention on the GPU's own table (Z18 reading: decouples selection from attention)
    att = oracle.attend(w, x_host["q"], x_host["k"], x_host["v"], gp["idx"], gp["n_idx"])
    check_output(w, gp["out"].reshape(-1, w.head_dim), att["out"])
    lse_g = gp["lse"].t().reshape(-1).double().numpy()          # [h_q, total_q] -> (i, h) order
    assert np.abs(lse_g - att["lse"]).max() < lse_tol(w)
    # GPU attention on the oracle's own table
    sel = oracle.select(w, x_host["q"], kc, x_host["k"])
    idx_o, n_o = oracle.table(w, sel)
    p = gp["p"]
    out2 = sa.fwd(p, xg["q"], xg["k"], xg["v"], torch.from_numpy(idx_o).to(xg["q"].device),
                  torch.from_numpy(n_o).to(xg["q"].device))
    att2 = oracle.attend(w, x_host["q"], x_host["k"], x_host["v"], idx_o, n_o)
    check_output(w, out2.float().cpu().reshape(-1, w.head_dim), att2["out"], "output on oracle table")
    return dict(gpu=gp, flagged=n_flag)


def gen_pair(w, device="cuda", gen_on_device=False):
    """Inputs on host and device: generated on the host (small) or on the device (large)."""
    if gen_on_device:
        xg = generate(w, device=device)
        return to_host(xg), xg
    x = generate(w)
    return x, to_device(x, device)
