"""Host-side checks of bench.py (no GPU): the one-GPU contract and the work counts its
roofline figures are built on.

The attended-set sizes that price the attention (bytes for decode and drafts, flops for
prefill) are counted by bench.py from the selection table alone, edge blocks clipped in
closed form; here they must equal the oracle's own |A| per (query, head), which walks the
attended set position by position, on the oracle's tables for every small workload.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from workloads import FULL, generate, small

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", list(FULL))
def test_attended_totals_match_the_oracle(name):
    w = small(name)
    x = generate(w)
    kc = oracle.compress(w, x["k"]) if w.block > 1 else None
    sel = oracle.select(w, x["q"], kc, x["k"])
    idx, n = oracle.table(w, sel)
    cnt = oracle.attend(w, x["q"], x["k"], x["v"], idx, n)["count"].reshape(w.total_q, w.h_q)
    per_qkv = cnt[:, ::w.h_q // w.h_kv]                  # the group's heads share one set
    assert (cnt.reshape(w.total_q, w.h_kv, -1) == per_qkv[:, :, None]).all()
    assert bench.attended_total_exact(w, idx, n) == int(per_qkv.sum())
    if w.shared_selection:
        # once per (sequence, KV head), with the largest of its drafts' sets
        q_off = np.cumsum([0] + list(w.seqlens_q))
        want = sum(int(per_qkv[q_off[b]:q_off[b + 1], c].max()) for b in range(w.batch) for c in range(w.h_kv))
        assert bench.attended_total_exact(w, idx, n, per_unit=True) == want


def test_next_rows_name_real_options():
    """Every variant the default line measures names a workload, options the script parses
    and workload fields that exist."""
    import dataclasses
    dests = {a.dest for a in bench.arg_parser()._actions}
    fields = {f.name for f in dataclasses.fields(FULL["bf16_decode_32k"]())}
    assert {"page_size", "lsa_buckets", "s3r_refresh", "no_cpu_baseline"} <= dests
    for key, name, opts, wfields in bench.NEXT_ROWS:
        assert name in FULL, key
        assert set(opts) <= dests, key
        assert set(wfields) <= fields, key
        assert FULL[name]().scaled(**wfields).name == name
