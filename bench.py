"""Benchmark of the selector-driven top-k sparse attention hot path on one MI355X.

Default workload: bf16 decode, 32 sequences x 32768 cached tokens, Hq 32 / Hkv 8,
d 128, g 64, top-32 blocks + 1 init block + 128-token window.  One step is the
whole path for one decode token per sequence: re-pool the newest block of every
sequence (sparse_attn_compress_tail), select (sparse_attn_select) and attend
(sparse_attn_fwd).  Inputs are synthetic and already resident in HBM.

Prints one JSON line.  ``--workload`` runs one of the other synthetic workloads
instead (prefill workloads report tok/s).
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
from workloads import DTYPE_BF16, FULL, generate, hot_blocks  # noqa: E402

METRIC = "sparse-attn prefill tok/s + decode µs/step; % HBM GB/s / % MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DECODE = ("bf16_decode_32k", "bf16_draft_decode")


def make_params(w, device):
    dt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32
    return sa.Params.from_lengths(w.seqlens_q, w.seqlens_k, device=device, h_q=w.h_q, h_kv=w.h_kv,
                                  head_dim=w.head_dim, block=w.block, pool=w.pool, topk=w.topk,
                                  n_init=w.n_init, window=w.window, shared_selection=w.shared_selection,
                                  topk_per_seq=w.topk_per_seq, dtype=dt)


class TimingEvents:
    """HIP events for the attention kernel's live duration, created with
    hipEventDisableSystemFence: a default event's record performs a system-scope
    release (cache write-back) between the kernels of the step, which costs several
    microseconds per record in a decode step and is not needed to read a timestamp.
    They live in the HIP runtime the process already loaded (torch's)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                ev = ctypes.c_void_p()
                rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
                if rc != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
                pair.append(ev.value)
            self.pairs.append(tuple(pair))

    def mean_ms(self):
        tot = 0.0
        for a, b in self.pairs:
            ms = ctypes.c_float()
            rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            tot += ms.value
        return tot / len(self.pairs)

    def close(self):
        for pair in self.pairs:
            for ev in pair:
                self.hip.hipEventDestroy(ev)
        self.pairs = []


class Step:
    """Preallocated buffers and the three ABI calls of one pass."""

    def __init__(self, w, x, device):
        self.w, self.x = w, x
        self.p = make_params(w, device)
        self.decode = w.name in DECODE
        sel_b, fwd_b = sa.workspace_size(self.p)
        self.ws_sel = torch.empty(max(sel_b, 16), dtype=torch.uint8, device=device)
        self.ws_fwd = torch.empty(max(fwd_b, 16), dtype=torch.uint8, device=device)
        self.k_cmp = torch.empty((w.h_kv, w.batch, self.p.nb_max, w.head_dim), dtype=torch.float32,
                                 device=device) if w.block > 1 else None
        self.idx = torch.empty((w.h_kv, self.p.rows, max(w.topk, 1)), dtype=torch.int32, device=device)
        self.n_idx = torch.empty((w.h_kv, self.p.rows), dtype=torch.int32, device=device)
        self.out = torch.empty_like(x["q"])
        if self.k_cmp is not None and self.decode:
            sa.compress(self.p, x["k"], self.k_cmp)       # the cache's pooled keys, built before decoding

    def __call__(self, events=None):
        x = self.x
        if self.k_cmp is not None:
            if self.decode:
                sa.compress_tail(self.p, 1, x["k"], self.k_cmp)
            else:
                sa.compress(self.p, x["k"], self.k_cmp)
        sa.select(self.p, x["q"], self.k_cmp, x["k"], self.idx, self.n_idx, ws=self.ws_sel)
        sa.fwd(self.p, x["q"], x["k"], x["v"], self.idx, self.n_idx, out=self.out, ws=self.ws_fwd,
               events=events)


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


# Dominant kernel of each workload and the sources it is built from: a counter record
# is used only while these files are unchanged.
CSRC = "top_block_sparse_mean_amd/csrc/"
KERNEL_SOURCES = {
    "sa::attn_mfma_kernel": [CSRC + "attn_decode.hip", CSRC + "mfma_common.hpp", CSRC + "sa_common.hpp",
                             CSRC + "sa_internal.hpp"],
    "sa::attn_wg_kernel": [CSRC + "attn_prefill.hip", CSRC + "mfma_common.hpp", CSRC + "sa_common.hpp",
                           CSRC + "sa_internal.hpp"],
}
DOMINANT = {"bf16_decode_32k": "sa::attn_mfma_kernel", "bf16_prefill_128k": "sa::attn_wg_kernel"}


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


def cpu_baseline(w, x, seconds=10.0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    oracle.lib()
    nb = 2 if w.name in DECODE else 1
    if w.name == "bf16_decode_32k":
        sub = w.scaled(seqlens_k=w.seqlens_k[:nb], seqlens_q=w.seqlens_q[:nb])
        xs = {k: x[k][:sum(sub.seqlens_q if k == "q" else sub.seqlens_k)].cpu().contiguous()
              for k in ("q", "k", "v")}
        kc = oracle.compress(sub, xs["k"])
        reps, t0 = 0, time.perf_counter()
        while True:
            sel = oracle.select(sub, xs["q"], kc, xs["k"])
            idx, n = oracle.table(sub, sel)
            oracle.attend(sub, xs["q"], xs["k"], xs["v"], idx, n)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        per_seq_s = (time.perf_counter() - t0) / reps / nb
        return dict(value=per_seq_s * w.batch * 1e6, unit="µs/step", cores=oracle.num_threads(),
                    kind="oracle",
                    sample=f"select + attend of {nb} of {w.batch} sequences (all 8 KV heads, 32 query heads), "
                           f"{reps} repetitions, pooled keys precomputed; scaled x{w.batch // nb} to one step")
    # prefill workloads: a contiguous sample of query rows, scaled to the whole chunk
    kc = oracle.compress(w, x["k"].cpu()) if w.block > 1 else None
    xs = {k: x[k].cpu().contiguous() for k in ("q", "k", "v")}
    rng = np.random.default_rng(0)
    n_rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        rows = rng.integers(0, w.rows, size=8)
        sel = oracle.select(w, xs["q"], kc, xs["k"], rows=np.repeat(rows, w.h_kv),
                            heads=np.tile(np.arange(w.h_kv), 8))
        idx = np.full((w.h_kv, w.rows, sel["idx"].shape[1]), -1, dtype=np.int32)
        n = np.zeros((w.h_kv, w.rows), dtype=np.int32)
        idx[sel["heads"], sel["rows"]] = sel["idx"]
        n[sel["heads"], sel["rows"]] = sel["n"]
        reqs = np.repeat(rows, w.h_q)
        oracle.attend(w, xs["q"], xs["k"], xs["v"], idx, n, reqs=reqs, heads=np.tile(np.arange(w.h_q), 8))
        n_rows += 8
    el = time.perf_counter() - t0
    tok_s = n_rows / el
    return dict(value=tok_s, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"select + attend of {n_rows} random query rows (all heads), pooled keys precomputed")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_decode_32k", choices=sorted(FULL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a known-size kernel that "
                         "calibrates HBM byte counters in a profiled run)")
    ap.add_argument("--record-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write the workload's counter record under profiles/ from the output "
                         "directories of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script")
    args = ap.parse_args()
    if args.record_counters:
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
    w = FULL[args.workload]()
    x = generate(w, device=device)
    torch.cuda.synchronize()
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device=device).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step = Step(w, x, device)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    tev = TimingEvents(args.steps)
    evs = tev.pairs
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_begin.record()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(events=evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_begin.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    attn_ms = tev.mean_ms()
    tev.close()

    idx_h, n_h = step.idx.cpu().numpy(), step.n_idx.cpu().numpy()
    a_tot = attended_total_exact(w, idx_h, n_h)
    d = w.head_dim
    elt = 2 if w.dtype == DTYPE_BF16 else 4
    decode = w.name in DECODE
    if decode:
        a_read = attended_total_exact(w, idx_h, n_h, per_unit=True)
        attn_bytes = a_read * 2 * d * elt + 2 * w.total_q * w.h_q * d * elt
        roof = dict(bound="hbm", achieved=round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s")
        roof["frac"] = round(roof["achieved"] / HBM_PEAK_GBS, 4)
        value, unit, hib = ms_step * 1e3, "µs/step", False
    else:
        G = w.group
        flops = 4.0 * d * a_tot * G
        roof = dict(bound="mfma", achieved=round(flops / (attn_ms * 1e-3) / 1e12, 2), peak=BF16_PEAK_TFLOPS,
                    unit="TFLOP/s")
        roof["frac"] = round(roof["achieved"] / BF16_PEAK_TFLOPS, 4)
        value, unit, hib = w.total_q / (ms_step * 1e-3), "tok/s", True
        attn_bytes = None
    roof["traffic"] = measured_traffic(w.name)

    extra = {}
    if w.name == "bf16_decode_32k":
        hits = tot = 0
        for b in range(w.batch):
            for c in range(w.h_kv):
                hb = hot_blocks(w, b, c)
                sel = set(idx_h[c, b, :n_h[c, b]].tolist())
                hits += sum(1 for j in hb if j in sel)
                tot += len(hb)
        extra["hot_block_recall"] = round(hits / max(tot, 1), 4)

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": hib,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == DTYPE_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": d,
                   "max_k": w.max_k, "queries": w.total_q, "block": w.block, "topk": w.topk,
                   "n_init": w.n_init, "window": w.window, "parallelism": "single-gpu"},
        "roofline": roof,
        "attn_kernel_ms": round(attn_ms, 5),
        "attn_algorithmic_bytes": attn_bytes,
        "attended_tokens": a_tot,
        "wall_s": round(wall, 4),
        **extra,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, seconds=args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
