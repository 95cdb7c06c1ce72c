"""Benchmark of the selector-driven top-k sparse attention hot path on one MI355X.

Default workload: bf16 decode, 32 sequences x 32768 cached tokens, Hq 32 / Hkv 8,
d 128, g 64, top-32 blocks + 1 init block + 128-token window.  One step is the
whole path for one decode token per sequence: append its key and value to the
cache and re-pool the block it falls in (sparse_attn_append_kv), select
(sparse_attn_select) and attend (sparse_attn_fwd).  Inputs are synthetic and
already resident in HBM.

Prints one JSON line.  ``--workload`` runs one of the other synthetic workloads
instead (prefill workloads report tok/s); ``--page-size`` keeps K and V in a
paged cache.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import top_block_sparse_mean_amd as sa  # noqa: E402
from workloads import (DTYPE_BF16, FULL, from_pages, generate, hot_blocks, needle_groups,  # noqa: E402
                       page_layout, to_pages)

METRIC = "sparse-attn prefill tok/s + decode µs/step; % HBM GB/s / % MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
DECODE = ("bf16_decode_32k", "bf16_draft_decode")


def make_params(w, device, layout=None):
    dt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device=device, h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk,
                                  n_init=w.n_init, window=w.window, shared_selection=w.shared_selection,
                                  topk_per_seq=w.topk_per_seq, dtype=dt, pool_overlap=w.pool_overlap,
                                  select_mode=w.select_mode, select_tau=w.select_tau,
                                  block_table=None if layout is None else layout.block_table.to(device),
                                  page_size=0 if layout is None else layout.page_size)


class TimingEvents:
    """HIP events for the attention kernel's live duration, created with
    hipEventDisableSystemFence: a default event's record performs a system-scope
    release (cache write-back) between the kernels of the step, which costs several
    microseconds per record in a decode step and is not needed to read a timestamp.
    They live in the HIP runtime the process already loaded (torch's)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, width=2):
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            pair = []
            for _ in range(width):
                ev = ctypes.c_void_p()
                rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
                if rc != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
                pair.append(ev.value)
            self.pairs.append(tuple(pair))

    def record(self, ev):
        rc = self.hip.hipEventRecord(ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def mean_ms(self, i=0, j=1):
        """Mean over the recorded sets of the time from event i to event j."""
        return sum(self.elapsed_ms(evs[i], evs[j]) for evs in self.pairs) / len(self.pairs)

    def close(self):
        for pair in self.pairs:
            for ev in pair:
                self.hip.hipEventDestroy(ev)
        self.pairs = []


class Step:
    """Preallocated buffers and the ABI calls of one pass.  Prefill: compress, select,
    fwd.  Decode (one token per sequence) and draft rounds (the drafts of every
    sequence): append the new tokens' keys and values to the cache, which re-pools
    the blocks they fall in, then select and fwd.  The cache already holds those
    tokens, so every step rewrites the same values.  page_size > 0 keeps K and V in
    a paged cache read through a block table."""

    def __init__(self, w, x, device, page_size=0, buckets=False):
        self.w = w
        self.buckets = buckets
        self.layout = page_layout(w.seqlens_k, page_size, w.seed) if page_size else None
        if self.layout is not None:
            x = dict(x, k=to_pages(x["k"], self.layout), v=to_pages(x["v"], self.layout))
        self.x = x
        if buckets:          # the table holds the chosen buckets' groups: width = buckets x cap / g
            w = w.scaled(topk=w.bucket_topk * (w.bucket_cap // w.block))
            self.w = w
        self.p = make_params(w, device, self.layout)
        self.decode = w.name in DECODE
        # decode rows with the summed group score: the step is one sparse_attn_decode_step
        # call (append, select and attend in one launch); the kernel pass brackets that
        # launch.  The variant group scores run append+select, then fwd.
        self.fused_step = self.decode and not w.shared_selection and w.block > 1 and not buckets and \
            w.select_mode == 0
        # the kernel pass brackets the selection's scoring kernel (not with the bucket
        # index, nor when the step is one launch)
        self.time_select = not buckets and not self.fused_step
        self.index = sa.BucketIndex(self.p, w.bucket_block, w.bucket_count, w.bucket_cap) if buckets else None
        sel_b, fwd_b = sa.workspace_size(self.p)
        self.ws_sel = torch.empty(max(sel_b, 16), dtype=torch.uint8, device=device)
        self.ws_fwd = torch.empty(max(fwd_b, 16), dtype=torch.uint8, device=device)
        self.ws_step = self.ws_sel if sel_b >= fwd_b else self.ws_fwd
        self.k_cmp = torch.empty((w.h_kv, w.batch, self.p.nb_max, w.head_dim), dtype=torch.float32,
                                 device=device) if w.block > 1 else None
        self.idx = torch.empty((w.h_kv, self.p.rows, max(w.topk, 1)), dtype=torch.int32, device=device)
        self.n_idx = torch.empty((w.h_kv, self.p.rows), dtype=torch.int32, device=device)
        self.out = torch.empty_like(x["q"])
        if buckets:
            # the history's buckets exist before the chunk arrives: build them once, untimed
            self.build_from = min(nk - nq for nk, nq in zip(w.seqlens_k, w.seqlens_q)) // w.bucket_block
            if self.k_cmp is not None:
                sa.compress(self.p, x["k"], self.k_cmp)
                sa.bucket_build(self.p, self.k_cmp, self.index)
            nb = ctypes.c_size_t(0)
            sa._lib.check("sparse_attn_bucket_workspace_size", sa.lib().sparse_attn_bucket_workspace_size(
                self.p.ref(), self.index.ref(), int(w.bucket_topk), ctypes.byref(nb)))
            self.ws_bkt = torch.empty(max(nb.value, 16), dtype=torch.uint8, device=device)
        if self.decode:
            # the new tokens: the last M_b of every sequence (packed rows of the generated K/V)
            new, o = [], 0
            for nk, nq in zip(w.seqlens_k, w.seqlens_q):
                new.extend(range(o + nk - nq, o + nk))
                o += nk
            rows = torch.tensor(new, device=device)
            src_k = x["k"] if self.layout is None else from_pages(x["k"], self.layout)
            src_v = x["v"] if self.layout is None else from_pages(x["v"], self.layout)
            self.k_new = src_k[rows].contiguous()
            self.v_new = src_v[rows].contiguous()
            if self.k_cmp is not None:
                sa.compress(self.p, x["k"], self.k_cmp)   # the cache's pooled keys, built before decoding

    def __call__(self, events=None):
        """events: four events, recorded around the selection's scoring kernel ([0], [1])
        and the main attention kernel ([2], [3]) -- around the one launch ([2], [3]) of a
        fused decode step."""
        x = self.x
        # decode: append + select in one call (one launch for decode rows), or the whole
        # step in one call
        joined = self.decode and self.index is None
        if self.decode and not joined:
            sa.append_kv(self.p, self.k_new, self.v_new, x["k"], x["v"], self.k_cmp)
        elif self.k_cmp is not None and not self.decode:
            sa.compress(self.p, x["k"], self.k_cmp)
            if self.index is not None:      # the chunk's new cluster blocks; earlier ones are frozen
                sa.bucket_build(self.p, self.k_cmp, self.index, build_from=self.build_from)
        if joined and self.fused_step:
            sa.decode_step(self.p, self.k_new, self.v_new, x["k"], x["v"], self.k_cmp, x["q"], self.idx, self.n_idx,
                           out=self.out, ws=self.ws_step, events=None if events is None else events[2:4])
            return
        if self.index is not None:
            sa.bucket_select(self.p, x["q"], self.index, self.w.bucket_topk, self.idx, self.n_idx, ws=self.ws_bkt)
        elif joined:
            sa.append_select(self.p, self.k_new, self.v_new, x["k"], x["v"], self.k_cmp, x["q"], self.idx, self.n_idx,
                             ws=self.ws_sel, events=events[0:2] if events is not None and self.time_select else None)
        else:
            sa.select(self.p, x["q"], self.k_cmp, x["k"], self.idx, self.n_idx, ws=self.ws_sel,
                      events=events[0:2] if events is not None and self.time_select else None)
        sa.fwd(self.p, x["q"], x["k"], x["v"], self.idx, self.n_idx, out=self.out, ws=self.ws_fwd,
               events=None if events is None else events[2:4])


    def stage(self, i):
        """One of the three calls a step is made of, alone (as the stage pass times them):
        0 compress (decode: append; with the bucket index: compress and the chunk's
        clustering), 1 select, 2 fwd.  Each rewrites the same values, so repeating one
        leaves the inputs of the others unchanged."""
        x = self.x
        if i == 0:
            if self.decode:
                sa.append_kv(self.p, self.k_new, self.v_new, x["k"], x["v"], self.k_cmp)
            elif self.k_cmp is not None:
                sa.compress(self.p, x["k"], self.k_cmp)
                if self.index is not None:
                    sa.bucket_build(self.p, self.k_cmp, self.index, build_from=self.build_from)
        elif i == 1:
            if self.index is not None:
                sa.bucket_select(self.p, x["q"], self.index, self.w.bucket_topk, self.idx, self.n_idx, ws=self.ws_bkt)
            else:
                sa.select(self.p, x["q"], self.k_cmp, x["k"], self.idx, self.n_idx, ws=self.ws_sel)
        else:
            sa.fwd(self.p, x["q"], x["k"], x["v"], self.idx, self.n_idx, out=self.out, ws=self.ws_fwd)


def attended_total_exact(w, idx_host, n_idx_host, per_unit=False):
    """Sum over (query, KV head) of the attended-set size |A|, edge blocks clipped exactly.
    per_unit: with a shared selection, count each (sequence, KV head) once with its largest
    set (the last draft's, which holds every other draft's) -- the positions the attention
    kernel reads once per unit."""
    import numpy as np
    tot = 0
    qi = 0
    g = w.block
    for b in range(w.batch):
        nk, nq = w.seqlens_k[b], w.seqlens_q[b]
        q0 = nk - nq
        p = np.arange(q0, nk)
        p_sel = np.full_like(p, q0 - 1) if w.shared_selection else p
        rows = np.full_like(p, b) if w.shared_selection else np.arange(qi, qi + nq)
        n1 = np.minimum(w.n_init, p + 1)
        hi = p_sel - w.window + 1
        lo_w = np.maximum(w.n_init, hi)
        n3 = np.maximum(0, p - lo_w + 1)
        for c in range(w.h_kv):
            ns = n_idx_host[c, rows]
            first = idx_host[c, rows, 0]
            last = idx_host[c, rows, np.maximum(ns - 1, 0)]
            f0 = np.maximum(first * g, w.n_init)
            lf = np.maximum(0, np.minimum(np.minimum((first + 1) * g, nk), hi) - f0)
            ll = np.maximum(0, np.minimum(np.minimum((last + 1) * g, nk), hi) - last * g)
            n2 = np.where(ns == 0, 0, np.where(ns == 1, lf, lf + (ns - 2) * g + ll))
            a = n1 + n2 + n3
            tot += int(a.max()) if (per_unit and w.shared_selection and len(a)) else int(a.sum())
        qi += nq
    return tot


def measured_peaks(device, prefill):
    """Achievable rates on this GPU, measured beside the published peaks: a 1 GiB
    device-to-device copy (GB/s, bytes read + written), a 2 GiB read-only reduction
    (GB/s read) and, for prefill workloads, 8192^3 library GEMMs in bf16 and fp32
    (TFLOP/s)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    out = {}
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    out["copy_gbs"] = round(2 * n * 4 / timed(lambda: dst.copy_(src), 20) / 1e9, 1)
    # read-only streaming: row sums of a 2 GiB [.., 4096] fp32 matrix (bytes read; the
    # ceiling of the read-only kernels: the decode gathers and the key scans).  Of the
    # library reductions tried this one reads fastest (a full reduction to one value
    # reached only ~4 TB/s)
    big = torch.empty((2 * n // 4096, 4096), dtype=torch.float32, device=device).fill_(1.0)
    acc = torch.empty(big.shape[0], dtype=torch.float32, device=device)
    out["read_gbs"] = round(2 * n * 4 / timed(lambda: torch.sum(big, dim=1, out=acc), 20) / 1e9, 1)
    del src, dst, big, acc
    if prefill:
        m = 8192
        for name, dt in (("bf16_gemm_tflops", torch.bfloat16), ("fp32_gemm_tflops", torch.float32)):
            a = torch.randn(m, m, device=device).to(dt)
            bm = torch.randn(m, m, device=device).to(dt)
            c = torch.empty(m, m, device=device, dtype=dt)
            out[name] = round(2.0 * m ** 3 / timed(lambda: torch.mm(a, bm, out=c), 5) / 1e12, 1)
            del a, bm, c
    torch.cuda.empty_cache()
    return out


def stage_report(w, stage_ms, attn_bytes, attn_flops, peaks, buckets=False):
    """Each stage of one step against its own bound, on algorithmic work.
    compress: keys read once + pooled keys written (HBM).  select: decode reads the
    pooled keys (or, with g = 1, the raw keys) once per step (HBM); prefill scores every
    causally visible block of every row per KV head (2 d flop each, fp32 MFMA).  fwd:
    the attention kernel's own figure (bytes for decode, useful flops for prefill)."""
    d, g = w.head_dim, w.block
    elt = 2 if w.dtype == DTYPE_BF16 else 4
    decode = w.name in DECODE
    nb = [-(-nk // g) for nk in w.seqlens_k]
    rep = {}

    def add(name, ms, amount, bound):
        r = {"ms": round(ms, 5), "bound": bound}
        if amount is not None and ms > 0:
            if bound == "hbm":
                r.update(achieved=round(amount / (ms * 1e-3) / 1e9, 1), unit="GB/s",
                         frac=round(amount / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         frac_of_measured=round(amount / (ms * 1e-3) / 1e9 / peaks["read_gbs"], 4))
            else:
                peak, mkey = (BF16_PEAK_TFLOPS, "bf16_gemm_tflops") if bound == "mfma_bf16" else \
                             (FP32_PEAK_TFLOPS, "fp32_gemm_tflops")
                ach = amount / (ms * 1e-3) / 1e12
                r.update(achieved=round(ach, 2), unit="TFLOP/s", frac=round(ach / peak, 4))
                if mkey in peaks:
                    r["frac_of_measured"] = round(ach / peaks[mkey], 4)
        rep[name] = r

    if buckets:
        # pooling, then Ward clustering of every cluster block (pair costs in LDS): no single bound
        add("index", stage_ms[0], None, "mixed")
    elif decode:
        # the new tokens' K/V rows written and their blocks re-pooled: launch-bound
        add("append", stage_ms[0], None, "launch")
    elif g > 1:
        add("compress", stage_ms[0], w.total_k * w.h_kv * d * elt + w.h_kv * sum(nb) * d * 4, "hbm")
    amount, bound = select_work(w, buckets)
    add("select", stage_ms[1], amount, bound)
    if decode:
        add("fwd", stage_ms[2], attn_bytes, "hbm")
    else:
        add("fwd", stage_ms[2], attn_flops, "mfma_bf16" if w.dtype == DTYPE_BF16 else "alu_fp32")
    return rep


def select_work(w, buckets=False):
    """Algorithmic work of the selection's scoring: decode rows read the pooled keys (or,
    with g = 1, the raw keys) once per step, plus the selector queries (bytes, HBM);
    prefill rows score every causally visible block of every row per KV head (2 d flop
    each, fp32 MFMA)."""
    d, g = w.head_dim, w.block
    elt = 2 if w.dtype == DTYPE_BF16 else 4
    if w.name in DECODE:
        nb = [-(-nk // g) for nk in w.seqlens_k]
        sel_bytes = (w.h_kv * sum(nb) * d * 4) if g > 1 else (w.h_kv * w.total_k * d * elt)
        return sel_bytes + w.total_q * w.h_q * d * elt, "hbm"
    cand = 0
    for nk, nq in zip(w.seqlens_k, w.seqlens_q):
        p = range(nk - nq, nk)
        if buckets:        # the centroids of the complete cluster blocks before each row
            cand += sum((q + 1) // w.bucket_block * w.bucket_count for q in p)
        else:
            cand += sum(q // g + 1 for q in p)
    return 2.0 * d * w.h_kv * cand, "mfma_fp32"


def needle_recall(w, idx_host, n_idx_host):
    """Fraction of the chunk's query rows in segment i whose selected groups hold needle
    group i, averaged over the planted needles (KV head 0)."""
    groups = needle_groups(w, 0)
    if not groups:
        return None
    fr = []
    for i, jg in enumerate(groups):
        r0, r1 = i * w.needle_segment, min((i + 1) * w.needle_segment, w.seqlens_q[0])
        hit = sum(1 for r in range(r0, r1) if jg in set(idx_host[0, r, :n_idx_host[0, r]].tolist()))
        fr.append(hit / (r1 - r0))
    return round(sum(fr) / len(fr), 4)


# Dominant kernel of each workload and the sources it is built from: a counter record
# is used only while these files are unchanged.
CSRC = "top_block_sparse_mean_amd/csrc/"
KERNEL_SOURCES = {
    "sa::attn_mfma_kernel": [CSRC + "attn_decode.hip", CSRC + "mfma_common.hpp", CSRC + "sa_common.hpp",
                             CSRC + "sa_internal.hpp"],
    "sa::decode_step_kernel": [CSRC + "select.hip", CSRC + "append_common.hpp", CSRC + "mfma_common.hpp",
                               CSRC + "sa_common.hpp", CSRC + "sa_internal.hpp"],
    "sa::attn_wg_kernel": [CSRC + "attn_prefill.hip", CSRC + "mfma_common.hpp", CSRC + "sa_common.hpp",
                           CSRC + "sa_internal.hpp"],
    "sa::score_rows_kernel": [CSRC + "select.hip", CSRC + "append_common.hpp", CSRC + "mfma_common.hpp",
                              CSRC + "sa_common.hpp", CSRC + "sa_internal.hpp"],
    "sa::score_tile3_kernel": [CSRC + "select.hip", CSRC + "append_common.hpp", CSRC + "mfma_common.hpp",
                               CSRC + "sa_common.hpp", CSRC + "sa_internal.hpp"],
    "sa::attn_valu_kernel": [CSRC + "attn.hip", CSRC + "sa_common.hpp", CSRC + "sa_internal.hpp"],
}
DOMINANT = {"bf16_decode_32k": "sa::decode_step_kernel", "bf16_prefill_128k": "sa::attn_wg_kernel",
            "bf16_draft_decode": "sa::score_rows_kernel", "bf16_chunked_prefill_1m": "sa::score_tile3_kernel",
            "tiny_fp32_prefill": "sa::attn_valu_kernel"}
# workloads whose step is dominated by the selection's scoring kernel (rocprofv3 kernel stats)
SELECT_DOMINANT = ("bf16_draft_decode", "bf16_chunked_prefill_1m")


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(HERE, f), "rb").read())
    return h.hexdigest()


def counter_record_path(kernel, workload):
    name = kernel.split("::")[-1].replace("_kernel", "")
    return os.path.join(HERE, "profiles", f"{name}_{workload}_counters.json")


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    record (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain
    1 GiB device copy), or None when there is no record for the workload or the kernel's
    sources have changed since the counters were taken."""
    kernel = DOMINANT.get(workload)
    if kernel is None:
        return None
    path = counter_record_path(kernel, workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload or rec.get("sources_sha256") != sources_sha256(rec["sources"]):
        return None
    kib = (rec["fetch_kib_per_dispatch"] * rec["fetch_calibration"]["factor"]
           + rec["write_kib_per_dispatch"] * rec["write_calibration"]["factor"])
    return int(kib * 1024)


def record_counters(workload, fetch_dir, write_dir, commands):
    """Write the counter record of the workload's dominant kernel from two rocprofv3
    --pmc runs of this script with --copy-probe-mib 1024 (FETCH_SIZE, then WRITE_SIZE)."""
    import csv
    import glob
    kernel = DOMINANT[workload]

    def load(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        rows = [r for f in files for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        mine = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].replace("void ", "").startswith(kernel)]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not mine or not copies:
            raise SystemExit(f"no {counter} rows for {kernel} or for the calibration copy in {d}")
        return sum(mine) / len(mine), max(copies)

    fetch, fetch_copy = load(fetch_dir, "FETCH_SIZE")
    write, write_copy = load(write_dir, "WRITE_SIZE")
    expected = 1024 * 1024                          # KiB moved each way by the 1 GiB copy
    srcs = KERNEL_SOURCES[kernel]
    rec = {
        "kernel": kernel, "workload": workload, "sources": srcs, "sources_sha256": sources_sha256(srcs),
        "fetch_kib_per_dispatch": round(fetch, 2), "write_kib_per_dispatch": round(write, 2),
        "fetch_calibration": {"kernel": "__amd_rocclr_copyBuffer (1 GiB device copy)", "expected_kib": expected,
                              "counted_kib": fetch_copy, "factor": round(expected / fetch_copy, 4)},
        "write_calibration": {"kernel": "__amd_rocclr_copyBuffer (1 GiB device copy)", "expected_kib": expected,
                              "counted_kib": write_copy, "factor": round(expected / write_copy, 4)},
        "commands": commands,
    }
    path = counter_record_path(kernel, workload)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(path)


def s3r_refresh(w, step, steps, device):
    """The rest of an S3R round after the drafts (S3R review): the dense verify pass over
    the history and the drafts (a table keeping every candidate; attention with lse),
    then the next round's selection by the attention mass that pass put on each history
    token (select_mode SA_SELECT_ATTN).  Each leg is timed with events over `steps`
    repetitions; bytes are the keys and values read once per (sequence, KV head)."""
    from workloads import SELECT_ATTN
    x = step.x
    wd = w.scaled(topk=max(w.seqlens_k), topk_per_seq=None)
    pd = make_params(wd, device, step.layout)
    pa = make_params(w.scaled(select_mode=SELECT_ATTN), device, step.layout)
    sel_b, fwd_b = sa.workspace_size(pd)
    ws_sel = torch.empty(max(sel_b, 16), dtype=torch.uint8, device=device)
    ws_fwd = torch.empty(max(fwd_b, 16), dtype=torch.uint8, device=device)
    idx_d, n_d = sa.select(pd, x["q"], None, x["k"], ws=ws_sel)          # every candidate: dense
    ws_a = torch.empty(max(sa.workspace_size(pa)[0], 16), dtype=torch.uint8, device=device)
    out = torch.empty_like(x["q"])
    lse = torch.empty((w.h_q, w.total_q), dtype=torch.float32, device=device)
    idx = torch.empty((w.h_kv, pa.rows, max(w.topk, 1)), dtype=torch.int32, device=device)
    n_idx = torch.empty((w.h_kv, pa.rows), dtype=torch.int32, device=device)
    ev = TimingEvents(steps, width=3)

    def leg(evs=None):
        if evs:
            ev.record(evs[0])
        sa.fwd(pd, x["q"], x["k"], x["v"], idx_d, n_d, out=out, lse=lse, want_lse=True, ws=ws_fwd)
        if evs:
            ev.record(evs[1])
        sa.select(pa, x["q"], None, x["k"], idx, n_idx, ws=ws_a, attn_lse=lse)
        if evs:
            ev.record(evs[2])
    for _ in range(3):
        leg()
    torch.cuda.synchronize()
    for i in range(steps):
        leg(ev.pairs[i])
    torch.cuda.synchronize()
    v_ms, r_ms = ev.mean_ms(0, 1), ev.mean_ms(1, 2)
    ev.close()
    elt = 2 if w.dtype == DTYPE_BF16 else 4
    kv_bytes = w.total_k * w.h_kv * w.head_dim * elt
    return {"verify_ms": round(v_ms, 5), "refresh_ms": round(r_ms, 5),
            "verify_gbs": round(2 * kv_bytes / (v_ms * 1e-3) / 1e9, 1),
            "refresh_gbs": round(kv_bytes / (r_ms * 1e-3) / 1e9, 1),
            "round_us": None}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, seconds=10.0):
    """The oracle, as it stands, on a bounded sample of the same workload, timed stage by
    stage (compress, select, attend) on the host cores."""
    import numpy as np

    import oracle
    oracle.lib()
    clock = time.perf_counter
    if w.name in DECODE:
        nb = 2 if w.name == "bf16_decode_32k" else 4
        sub = w.scaled(seqlens_k=w.seqlens_k[:nb], seqlens_q=w.seqlens_q[:nb],
                       topk_per_seq=w.topk_per_seq[:nb] if w.topk_per_seq else w.topk_per_seq)
        xs = {k: x[k][:sum(sub.seqlens_q if k == "q" else sub.seqlens_k)].cpu().contiguous()
              for k in ("q", "k", "v")}
        t = clock()
        kc = oracle.compress(sub, xs["k"]) if w.block > 1 else None
        t_cmp = clock() - t
        reps, t_sel, t_att = 0, 0.0, 0.0
        while t_sel + t_att < seconds:
            t = clock()
            sel = oracle.select(sub, xs["q"], kc, xs["k"])
            idx, n = oracle.table(sub, sel)
            t2 = clock()
            oracle.attend(sub, xs["q"], xs["k"], xs["v"], idx, n)
            t_sel += t2 - t
            t_att += clock() - t2
            reps += 1
        # the work of a sequence grows with its cached length: scale by cached tokens
        grow = w.total_k / sub.total_k
        scale = grow / reps
        stages = {"select": round(t_sel * scale * 1e6, 1), "attend": round(t_att * scale * 1e6, 1)}
        if kc is not None:
            stages["compress_whole_cache"] = round(t_cmp * grow * 1e6, 1)
        return dict(value=(t_sel + t_att) * scale * 1e6, unit="µs/step", cores=oracle.num_threads(),
                    kind="oracle", cpu_model=cpu_model(), stages_us=stages,
                    sample=f"select + attend of the first {nb} of {w.batch} sequences (all {w.h_kv} KV heads, "
                           f"{w.h_q} query heads), {reps} repetitions, scaled x{grow:.1f} by cached tokens to "
                           f"one step" + ("; the step's re-pooling of one block per sequence is not timed (the "
                                          "whole cache's pooling is shown apart)" if kc is not None else ""))
    # prefill workloads: the whole compress, then random query rows, scaled to the whole chunk
    xs = {k: x[k].cpu().contiguous() for k in ("q", "k", "v")}
    t_cmp = 0.0
    kc = None
    if w.block > 1:
        t = clock()
        kc = oracle.compress(w, xs["k"])
        t_cmp = clock() - t
    rng = np.random.default_rng(0)
    n_rows, t_sel, t_att = 0, 0.0, 0.0
    while t_sel + t_att < seconds:
        rows = rng.integers(0, w.rows, size=8)
        t = clock()
        sel = oracle.select(w, xs["q"], kc, xs["k"], rows=np.repeat(rows, w.h_kv),
                            heads=np.tile(np.arange(w.h_kv), 8))
        idx = np.full((w.h_kv, w.rows, sel["idx"].shape[1]), -1, dtype=np.int32)
        n = np.zeros((w.h_kv, w.rows), dtype=np.int32)
        idx[sel["heads"], sel["rows"]] = sel["idx"]
        n[sel["heads"], sel["rows"]] = sel["n"]
        t2 = clock()
        reqs = np.repeat(rows, w.h_q)
        oracle.attend(w, xs["q"], xs["k"], xs["v"], idx, n, reqs=reqs, heads=np.tile(np.arange(w.h_q), 8))
        t_sel += t2 - t
        t_att += clock() - t2
        n_rows += 8
    scale = w.total_q / n_rows
    total_s = t_cmp + (t_sel + t_att) * scale
    return dict(value=w.total_q / total_s, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model(),
                stages_s={"compress": round(t_cmp, 3), "select": round(t_sel * scale, 3),
                          "attend": round(t_att * scale, 3)},
                sample=f"the whole compress once, then select + attend of {n_rows} random query rows "
                       f"(all heads), scaled x{scale:.1f} to the chunk")


def bench_workload(w, args, device, peaks, headline):
    """One workload at full size: W untimed steps, K timed steps bracketed by two events
    (nothing else recorded inside), then a kernel pass of the same steps with events
    around the selection's scoring kernel and the attention kernel (their launch
    durations, on the stream they run on), a stage pass (each call of the step repeated
    alone between two events), and the oracle on a bounded sample.  Returns the
    workload's figures."""
    x = generate(w, device=device)
    torch.cuda.synchronize()
    if args.copy_probe_mib and headline:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device=device).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step = Step(w, x, device, page_size=args.page_size if headline else 0,
                buckets=args.lsa_buckets and headline)
    w = step.w
    buckets = step.index is not None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_begin.record()
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_begin.elapsed_time(t_end) / args.steps

    # kernel pass: the same steps, with events around the two kernels that read the data
    n_k = max(1, min(args.steps, 20))
    kev = TimingEvents(n_k, width=4)
    for i in range(n_k):
        step(events=kev.pairs[i])
    torch.cuda.synchronize()
    attn_ms = kev.mean_ms(2, 3)
    bracket_ms = attn_ms
    if step.fused_step:
        # the step is that one launch: the timed steps' mean (launch plus the gap to the
        # next) and the bracketed launches' mean are both upper bounds of its duration.
        # The events around this launch read about 4 us above it (rocprofv3 sees the
        # bracketed launches run no longer than the others), so the smaller is used
        attn_ms = min(attn_ms, ms_step)
    score_ms = kev.mean_ms(0, 1) if step.time_select else None
    kev.close()

    # per-stage times: each of the three calls repeated n_k times back to back between two
    # events (events between the calls of a step would also time the host's launch gaps
    # once the recording host falls behind the GPU)
    sev = TimingEvents(3, width=2)
    stage_ms = []
    for i in range(3):
        step.stage(i)                                  # warm
        sev.record(sev.pairs[i][0])
        for _ in range(n_k):
            step.stage(i)
        sev.record(sev.pairs[i][1])
        torch.cuda.synchronize()
        stage_ms.append(sev.elapsed_ms(*sev.pairs[i]) / n_k)
    sev.close()

    idx_h, n_h = step.idx.cpu().numpy(), step.n_idx.cpu().numpy()
    a_tot = attended_total_exact(w, idx_h, n_h)
    d = w.head_dim
    elt = 2 if w.dtype == DTYPE_BF16 else 4
    decode = w.name in DECODE
    sel_amount, sel_bound = select_work(w, buckets)
    if decode:
        a_read = attended_total_exact(w, idx_h, n_h, per_unit=True)
        attn_bytes = a_read * 2 * d * elt + 2 * w.total_q * w.h_q * d * elt
        # one launch per step: its bytes are the pooled keys and the gathered K/V together
        roof_bytes = attn_bytes + (sel_amount if step.fused_step else 0)
        roof = dict(bound="hbm", achieved=round(roof_bytes / (attn_ms * 1e-3) / 1e9, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s")
        roof["frac"] = round(roof["achieved"] / HBM_PEAK_GBS, 4)
        roof["measured_peak"] = peaks["read_gbs"]
        roof["frac_of_measured"] = round(roof["achieved"] / peaks["read_gbs"], 4)
        roof["algorithmic_bytes"] = int(roof_bytes)
        value, unit, hib = ms_step * 1e3, "µs/step", False
        flops = None
    else:
        G = w.group
        flops = 4.0 * d * a_tot * G
        # bf16 runs on the matrix cores; the fp32 path's attention runs on the vector ALU
        peak = BF16_PEAK_TFLOPS if w.dtype == DTYPE_BF16 else FP32_PEAK_TFLOPS
        roof = dict(bound="mfma" if w.dtype == DTYPE_BF16 else "alu",
                    achieved=round(flops / (attn_ms * 1e-3) / 1e12, 2), peak=peak, unit="TFLOP/s")
        roof["frac"] = round(roof["achieved"] / peak, 4)
        if w.dtype == DTYPE_BF16:
            roof["measured_peak"] = peaks["bf16_gemm_tflops"]
            roof["frac_of_measured"] = round(roof["achieved"] / peaks["bf16_gemm_tflops"], 4)
        value, unit, hib = w.total_q / (ms_step * 1e-3), "tok/s", True
        attn_bytes = None
    kname = "sa::attn_mfma_kernel" if (buckets or (decode and not step.fused_step)) else \
        DOMINANT.get(w.name, "attention")
    roof = {"kernel": kname, **roof}
    if w.name in SELECT_DOMINANT and score_ms and not buckets:
        # the selection's scoring kernel dominates these steps: the roofline is its own,
        # the attention kernel's figure is kept beside it
        attn_roof = {k: v for k, v in roof.items() if k != "kernel"}
        attn_roof["kernel"] = "sa::attn_mfma_kernel"
        if sel_bound == "hbm":
            ach = sel_amount / (score_ms * 1e-3) / 1e9
            roof = dict(kernel=DOMINANT[w.name], bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                        unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), measured_peak=peaks["read_gbs"],
                        frac_of_measured=round(ach / peaks["read_gbs"], 4))
        else:
            ach = sel_amount / (score_ms * 1e-3) / 1e12
            roof = dict(kernel=DOMINANT[w.name], bound="mfma", dtype="fp32", achieved=round(ach, 2),
                        peak=FP32_PEAK_TFLOPS, unit="TFLOP/s", frac=round(ach / FP32_PEAK_TFLOPS, 4),
                        measured_peak=peaks["fp32_gemm_tflops"],
                        frac_of_measured=round(ach / peaks["fp32_gemm_tflops"], 4))
        roof["attention"] = attn_roof
    roof["traffic"] = None if buckets else measured_traffic(w.name)

    out = {"workload": w.name, "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_step, 5),
           "higher_is_better": hib, "dtype": "bf16" if w.dtype == DTYPE_BF16 else "f32",
           "config": {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": d,
                      "max_k": w.max_k, "queries": w.total_q, "block": w.block, "topk": w.topk,
                      "n_init": w.n_init, "window": w.window,
                      "kv_layout": f"paged{args.page_size}" if (args.page_size and headline) else "packed",
                      "select_mode": {0: "sum", 1: "softmax", 2: "max"}[w.select_mode],
                      "pool_overlap": w.pool_overlap, "selector": "lsa_buckets" if buckets else "blocks",
                      **({"append": "sparse_attn_append_select (one launch for decode rows)"} if decode else {}),
                      "parallelism": "single-gpu"},
           "roofline": roof}
    out["step_kernel_ms" if step.fused_step else "attn_kernel_ms"] = round(attn_ms, 5)
    if step.fused_step:
        out["bracketed_kernel_ms"] = round(bracket_ms, 5)
    if score_ms:
        out["score_kernel_ms"] = round(score_ms, 5)
    if step.fused_step:
        # the step's one launch reads the pooled keys and the gathered K/V
        out["select_plus_attn"] = {"bytes": int(sel_amount + attn_bytes), "kernel_ms": round(attn_ms, 5),
                                   "kernel": "sa::decode_step_kernel", "bound": "hbm",
                                   "achieved": roof["achieved"], "unit": "GB/s", "frac": roof["frac"],
                                   "frac_of_measured": roof["frac_of_measured"]}
    elif decode and score_ms and sel_bound == "hbm":
        # the two kernels that read the step's data, by their launch durations
        tot = sel_amount + attn_bytes
        ach = tot / ((score_ms + attn_ms) * 1e-3) / 1e9
        out["select_plus_attn"] = {"bytes": int(tot), "kernel_ms": round(score_ms + attn_ms, 5), "bound": "hbm",
                                   "achieved": round(ach, 1), "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                   "frac_of_measured": round(ach / peaks["read_gbs"], 4)}
    out["attn_algorithmic_bytes"] = attn_bytes
    out["attended_tokens"] = a_tot
    out["wall_s"] = round(wall, 4)
    if w.name == "bf16_decode_32k":
        hits = tot = 0
        for b in range(w.batch):
            for c in range(w.h_kv):
                hb = hot_blocks(w, b, c)
                sel = set(idx_h[c, b, :n_h[c, b]].tolist())
                hits += sum(1 for j in hb if j in sel)
                tot += len(hb)
        out["hot_block_recall"] = round(hits / max(tot, 1), 4)
    if w.structure == "needles":
        out["needle_recall"] = needle_recall(w, idx_h, n_h)
    if w.name == "bf16_draft_decode":
        out["us_per_draft_token"] = round(ms_step * 1e3 / w.seqlens_q[0], 3)
    out["stages"] = stage_report(w, stage_ms, attn_bytes, flops, peaks, buckets=buckets)
    if args.s3r_refresh and w.shared_selection and headline:
        r = s3r_refresh(w, step, min(args.steps, 20), device)
        r["round_us"] = round(ms_step * 1e3 + (r["verify_ms"] + r["refresh_ms"]) * 1e3, 2)
        out["s3r"] = r
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, seconds=args.cpu_seconds)
    del step, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# The metric is quoted on the decode step (the line's value) and the prefill rates; the
# draft round is the other decode-shaped workload.  The tiny fp32 workload is a parity case.
SECONDARY = ("bf16_prefill_128k", "bf16_chunked_prefill_1m", "bf16_draft_decode")

# The pieces that come after the path, each at full size on the workload it serves: a
# paged cache, the selector variants, the LSA bucket index and the rest of an S3R round
# (name: workload, option overrides, workload field overrides).
NEXT_ROWS = (
    ("paged16_decode", "bf16_decode_32k", {"page_size": 16}, {}),
    ("select_max_decode", "bf16_decode_32k", {}, {"select_mode": 2}),
    ("select_softmax_decode", "bf16_decode_32k", {}, {"select_mode": 1}),
    ("pool_overlap32_decode", "bf16_decode_32k", {}, {"pool_overlap": 32}),
    ("lsa_buckets_1m", "bf16_chunked_prefill_1m", {"lsa_buckets": True}, {}),
    ("s3r_round", "bf16_draft_decode", {"s3r_refresh": True}, {}),
)


def next_rows(args, device, peaks):
    """The NEXT_ROWS variants, each one bench_workload run without the oracle baseline;
    per row its value, its dominant kernel's roofline and, for the S3R round, the verify
    and refresh legs."""
    rows = {}
    for key, name, opts, fields in NEXT_ROWS:
        a = argparse.Namespace(**{**vars(args), "page_size": 0, "lsa_buckets": False, "s3r_refresh": False,
                                  "copy_probe_mib": 0, "no_cpu_baseline": True, **opts})
        r = bench_workload(FULL[name]().scaled(**fields), a, device, peaks, headline=True)
        print(f"# {key}: {r['value']} {r['unit']}", file=sys.stderr, flush=True)
        roof = r["roofline"]
        row = {"workload": name, "value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
               "config": {k: r["config"][k] for k in ("kv_layout", "select_mode", "pool_overlap", "selector")},
               "roofline": {k: roof.get(k) for k in ("kernel", "bound", "achieved", "peak", "unit", "frac")}}
        if "select_plus_attn" in r:
            row["select_plus_attn_frac"] = r["select_plus_attn"]["frac"]
        if "s3r" in r:
            row["s3r"] = r["s3r"]
        rows[key] = row
    return rows


def arg_parser():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(FULL),
                    help="run this workload alone (default: the decode step as the line's value, with the "
                         "128K prefill, the 1M-token chunk and the draft round beside it)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="keep K and V in a paged cache of this many tokens per page (0: packed)")
    ap.add_argument("--select-mode", choices=["sum", "softmax", "max"], default="sum",
                    help="group score of the selector: heads summed (default), sum of per-head softmaxes, "
                         "max over heads")
    ap.add_argument("--pool-overlap", type=int, default=0,
                    help="pooling windows reach this many tokens before their block (0: disjoint)")
    ap.add_argument("--lsa-buckets", action="store_true",
                    help="prefill workloads: select through the LSA flat bucket index (cluster blocks of 512 "
                         "tokens, 64 buckets of at most 16 tokens; 256 buckets per query); a step clusters the "
                         "blocks its chunk completes, the history's buckets are built beforehand")
    ap.add_argument("--s3r-refresh", action="store_true",
                    help="draft workload: also time the dense verify pass and the refreshed selection")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a known-size kernel that "
                         "calibrates HBM byte counters in a profiled run)")
    ap.add_argument("--record-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write the workload's counter record under profiles/ from the output "
                         "directories of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script")
    return ap


def main():
    args = arg_parser().parse_args()
    if args.record_counters:
        if args.workload is None:
            raise SystemExit("--record-counters needs --workload")
        cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d $REPO/{d} -o run "
               "-- python3 $REPO/bench.py --workload {w} --steps 5 --warmup 2 --no-cpu-baseline "
               "--copy-probe-mib 1024")
        record_counters(args.workload, *args.record_counters,
                        [cmd.format(c="FETCH_SIZE", d=args.record_counters[0], w=args.workload),
                         cmd.format(c="WRITE_SIZE", d=args.record_counters[1], w=args.workload)])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    device = "cuda"
    torch.cuda.set_device(0)
    name = args.workload or "bf16_decode_32k"
    others = [] if args.workload else list(SECONDARY)
    peaks = measured_peaks(device, prefill=True)
    w = FULL[name]().scaled(select_mode={"sum": 0, "softmax": 1, "max": 2}[args.select_mode],
                            pool_overlap=args.pool_overlap)
    head = bench_workload(w, args, device, peaks, headline=True)
    print(f"# {name}: {head['value']} {head['unit']}", file=sys.stderr, flush=True)
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": head["higher_is_better"],
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        **{k: v for k, v in head.items() if k not in ("workload", "value", "unit", "ms_per_step",
                                                       "higher_is_better", "dtype")},
        "measured_peaks": peaks,
    }
    prefill, other = {}, {}
    for o in others:
        r = bench_workload(FULL[o](), args, device, peaks, headline=False)
        print(f"# {o}: {r['value']} {r['unit']}", file=sys.stderr, flush=True)
        (prefill if r["unit"] == "tok/s" else other)[o] = r
    if prefill:
        res["prefill"] = prefill
    if other:
        res["other_decode"] = other
    if not args.workload:
        res["next_rows"] = next_rows(args, device, peaks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
