"""Seeded synthetic inputs for the workloads in ``configs.py``.

Everything is drawn with ``torch.Generator`` streams seeded from the
workload's seed and a per-tensor tag, in fp32, then rounded to the workload's
element type (bf16 by round-to-nearest-even).  The same tensors feed the HIP
path and the CPU oracle: they are generated once and copied to the other side.

Planted structure (input structure only, none of the method's arithmetic):
  * hot_blocks: per (sequence, KV head), ``n_hot`` distinct key blocks outside
    the sink and window get every key shifted by ``hot_shift`` along the unit
    direction of the group's summed query.
  * lowrank: per KV head an orthonormal basis U (QR of a Gaussian, d x r); per
    g-token block independent key and query latents a ~ N(0, I_r); keys and
    the group's queries of that block get ``scale*sqrt(d/r)*U a`` added.
  * needles: unit directions u_i planted (x needle_shift) on the raw keys of
    distinct pooled groups outside the sink and windows, and on every head of
    the queries of chunk segment i (``needle_segment`` consecutive queries).
"""
from __future__ import annotations

import hashlib

import torch

from .configs import DTYPE_BF16, Workload


def _gen(seed: int, tag: str, device) -> torch.Generator:
    h = int.from_bytes(hashlib.sha256(f"{seed}:{tag}".encode()).digest()[:7], "little")
    g = torch.Generator(device=device)
    g.manual_seed(h)
    return g


def _randn(shape, seed, tag, device):
    return torch.randn(shape, generator=_gen(seed, tag, device), device=device, dtype=torch.float32)


def _perm(n, seed, tag):
    return torch.randperm(n, generator=_gen(seed, tag, "cpu"))


def cu_seqlens(lens):
    out = [0]
    for x in lens:
        out.append(out[-1] + int(x))
    return torch.tensor(out, dtype=torch.int32)


def generate(w: Workload, device="cpu"):
    """Return dict(q, k, v, cu_q, cu_k, q0) for workload ``w`` on ``device``.

    q: [sum M_b, Hq, d], k/v: [sum N_b, Hkv, d] in the workload's dtype;
    cu_q/cu_k: int32 [batch+1] (on ``device``); q0: python list of the absolute
    position of each sequence's first query (right-aligned: N_b - M_b).
    """
    d, hq, hkv, G = w.head_dim, w.h_q, w.h_kv, w.group
    q = _randn((w.total_q, hq, d), w.seed, "q", device)
    k = _randn((w.total_k, hkv, d), w.seed, "k", device)
    v = _randn((w.total_k, hkv, d), w.seed, "v", device)
    cu_q = cu_seqlens(w.seqlens_q)
    cu_k = cu_seqlens(w.seqlens_k)
    q0 = [nk - nq for nk, nq in zip(w.seqlens_k, w.seqlens_q)]

    if w.structure == "hot_blocks":
        for b in range(w.batch):
            nk, qi = w.seqlens_k[b], int(cu_q[b + 1]) - 1
            hi = (nk - w.window) // w.block          # first block touching the window
            if hi <= 1:
                continue
            for c in range(hkv):
                n_hot = min(w.n_hot, hi - 1)
                blocks = (_perm(hi - 1, w.seed, f"hot:{b}:{c}")[:n_hot] + 1).tolist()
                u = q[qi, c * G:(c + 1) * G, :].sum(0)
                u = u / u.norm()
                base = int(cu_k[b])
                for j in blocks:
                    lo_t, hi_t = base + j * w.block, base + min((j + 1) * w.block, nk)
                    k[lo_t:hi_t, c, :] += w.hot_shift * u
    elif w.structure == "lowrank":
        r, g = w.lowrank_rank, w.block
        amp = w.lowrank_scale * (d / r) ** 0.5
        for b in range(w.batch):
            nk, nq = w.seqlens_k[b], w.seqlens_q[b]
            nblk = -(-nk // g)
            base_k, base_q = int(cu_k[b]), int(cu_q[b])
            tok_blk = torch.arange(nk, device=device) // g
            qpos_blk = (torch.arange(nq, device=device) + q0[b]) // g
            for c in range(hkv):
                basis, _ = torch.linalg.qr(_randn((d, r), w.seed, f"U:{b}:{c}", "cpu").double())
                basis = basis.float().to(device)
                ak = _randn((nblk, r), w.seed, f"aK:{b}:{c}", device)
                aq = _randn((nblk, r), w.seed, f"aQ:{b}:{c}", device)
                k[base_k:base_k + nk, c, :] += amp * (ak @ basis.T)[tok_blk]
                qshift = amp * (aq @ basis.T)[qpos_blk]
                q[base_q:base_q + nq, c * G:(c + 1) * G, :] += qshift[:, None, :]
    elif w.structure == "needles":
        g = w.block
        for b in range(w.batch):
            nk, nq = w.seqlens_k[b], w.seqlens_q[b]
            hi = (nk - nq - w.window) // g           # groups before every query's window
            n_seg = -(-nq // w.needle_segment)
            n = min(w.n_needles, n_seg, max(hi - 1, 0))
            if n == 0:
                continue
            groups = (_perm(hi - 1, w.seed, f"needle_groups:{b}")[:n] + 1).tolist()
            dirs = _randn((n, d), w.seed, f"needle_dirs:{b}", device)
            dirs = dirs / dirs.norm(dim=1, keepdim=True)
            base_k, base_q = int(cu_k[b]), int(cu_q[b])
            for i, jg in enumerate(groups):
                k[base_k + jg * g: base_k + min((jg + 1) * g, nk), :, :] += w.needle_shift * dirs[i]
                s0 = base_q + i * w.needle_segment
                s1 = base_q + min((i + 1) * w.needle_segment, nq)
                q[s0:s1, :, :] += w.needle_shift * dirs[i]
    elif w.structure != "iid":
        raise ValueError(w.structure)

    dt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                cu_q=cu_q.to(device), cu_k=cu_k.to(device), q0=q0)


def needle_groups(w: Workload, b: int = 0):
    """The planted needle groups of sequence b, in segment order (for recall reports)."""
    g = w.block
    nk, nq = w.seqlens_k[b], w.seqlens_q[b]
    hi = (nk - nq - w.window) // g
    n_seg = -(-nq // w.needle_segment)
    n = min(w.n_needles, n_seg, max(hi - 1, 0))
    if n == 0:
        return []
    return (_perm(hi - 1, w.seed, f"needle_groups:{b}")[:n] + 1).tolist()


def hot_blocks(w: Workload, b: int, c: int):
    """The planted hot blocks of (sequence b, KV head c) (for recall reports)."""
    nk = w.seqlens_k[b]
    hi = (nk - w.window) // w.block
    if hi <= 1:
        return []
    n_hot = min(w.n_hot, hi - 1)
    return sorted((_perm(hi - 1, w.seed, f"hot:{b}:{c}")[:n_hot] + 1).tolist())
