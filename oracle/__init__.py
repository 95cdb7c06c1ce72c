"""CPU fp64 oracle of selector-driven top-k sparse attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does: the two share no code.

The arithmetic lives in ``oracle.c`` (plain loops, double precision, OpenMP
over independent rows); this module only builds it with gcc and marshals
arguments.  Every function takes CPU tensors or numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build() -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math) into liboracle.so."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")      # a test may point at a deliberately broken build
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        L.or_compress.restype = ctypes.c_int
        L.or_select.restype = ctypes.c_int
        L.or_attend.restype = ctypes.c_int
        L.or_num_threads.restype = ctypes.c_int
        L.or_bucket_build.restype = ctypes.c_int
        L.or_bucket_select.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().or_num_threads()


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def _ptr(x, ctype=None):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        assert x.device.type == "cpu" and x.is_contiguous()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        p = x.data_ptr()
    else:
        assert x.flags["C_CONTIGUOUS"]
        p = x.ctypes.data
    return ctypes.cast(ctypes.c_void_p(p), ctype) if ctype else ctypes.c_void_p(p)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _geom(w, cu_q, cu_k, q_pos0):
    cu_q = _i32(cu_q if cu_q is not None else np.cumsum([0] + list(w.seqlens_q)))
    cu_k = _i32(cu_k if cu_k is not None else np.cumsum([0] + list(w.seqlens_k)))
    qp = None if q_pos0 is None else _i32(q_pos0)
    return cu_q, cu_k, qp


def compress(w, k, cu_k=None) -> np.ndarray:
    """Pooled keys K~ [Hkv, batch, nb_max, d] in fp64 (mean, or L2-normalised sum, over each
    block's window: its tokens and the w.pool_overlap tokens before them)."""
    _, cu_k, _ = _geom(w, None, cu_k, None)
    nb_max = -(-max(w.seqlens_k) // w.block)
    out = np.zeros((w.h_kv, w.batch, nb_max, w.head_dim), dtype=np.float64)
    rc = lib().or_compress(w.batch, w.h_kv, w.head_dim, _ptr(cu_k, _i32p), w.block, w.pool,
                           int(w.pool_overlap), w.dtype, _ptr(k), ctypes.c_int64(nb_max), _ptr(out, _f64p))
    assert rc == 0
    return out


def select_tau(w) -> float:
    """Softmax temperature of the SOFTMAX group score: the workload's, or sqrt(d)."""
    return float(w.select_tau) if w.select_tau > 0 else float(np.sqrt(w.head_dim))


def select(w, q_sel, k_cmp, k, rows=None, heads=None, q_pos0=None, cu_q=None, cu_k=None,
           topk_per_seq="workload", want_scores=False):
    """Selection for (row, KV head) requests; all rows x heads when ``rows`` is None.

    Returns dict(idx [n_req, kcap] int32 ascending and -1 padded, n [n_req],
    sk / sk1: the k-th and (k+1)-th scores in selection order (nan if absent),
    floor: the absolute near-tie floor, ncand: number of candidate blocks,
    rows, heads; scores [n_req, n_blocks] with nan for non-candidates if asked).
    """
    cu_q, cu_k, qp = _geom(w, cu_q, cu_k, q_pos0)
    n_rows = w.rows
    if rows is None:
        rr, hh = np.meshgrid(np.arange(n_rows), np.arange(w.h_kv), indexing="xy")
        heads = hh.reshape(-1)
        rows = rr.reshape(-1)
    rows, heads = _i64(rows), _i32(heads)
    n = len(rows)
    kcap = max(int(w.topk), 1)
    tps = w.topk_per_seq if topk_per_seq == "workload" else topk_per_seq
    tps = None if tps is None else _i32(tps)
    idx = np.empty((n, kcap), dtype=np.int32)
    nn = np.empty(n, dtype=np.int32)
    ncand = np.empty(n, dtype=np.int32)
    sk, sk1, fl = (np.empty(n, dtype=np.float64) for _ in range(3))
    nb_max = -(-max(w.seqlens_k) // w.block)
    if k_cmp is not None:
        k_cmp = np.ascontiguousarray(k_cmp, dtype=np.float64)
    n_blk = nb_max if w.block > 1 else max(w.seqlens_k)
    scores = np.full((n, n_blk), np.nan) if want_scores else None
    rc = lib().or_select(
        w.batch, w.h_q, w.h_kv, w.head_dim, _ptr(cu_q, _i32p), _ptr(cu_k, _i32p),
        _ptr(qp, _i32p), w.block, int(w.topk), _ptr(tps, _i32p), w.n_init, w.window,
        int(w.shared_selection), int(w.select_mode), ctypes.c_double(select_tau(w)), w.dtype, _ptr(q_sel),
        _ptr(k_cmp, _f64p),
        ctypes.c_int64(nb_max), _ptr(k), ctypes.c_int64(n), _ptr(rows, _i64p),
        _ptr(heads, _i32p), kcap, _ptr(idx, _i32p), _ptr(nn, _i32p), _ptr(sk, _f64p),
        _ptr(sk1, _f64p), _ptr(fl, _f64p), _ptr(ncand, _i32p), _ptr(scores, _f64p),
        ctypes.c_int64(n_blk))
    assert rc == 0, "selection exceeded the row capacity"
    return dict(idx=idx, n=nn, sk=sk, sk1=sk1, floor=fl, ncand=ncand, rows=rows, heads=heads,
                scores=scores)


def table(w, sel) -> tuple:
    """Scatter a full ``select`` result into [Hkv, rows, kcap] / [Hkv, rows] tables."""
    kcap = sel["idx"].shape[1]
    idx = np.full((w.h_kv, w.rows, kcap), -1, dtype=np.int32)
    n = np.zeros((w.h_kv, w.rows), dtype=np.int32)
    idx[sel["heads"], sel["rows"]] = sel["idx"]
    n[sel["heads"], sel["rows"]] = sel["n"]
    return idx, n


def attend(w, q, k, v, idx, n_idx, reqs=None, heads=None, scale=None, q_pos0=None, cu_q=None,
           cu_k=None, want_mask=False):
    """Attention over the attended set for (query, query-head) requests.

    idx [Hkv, rows, kcap] / n_idx [Hkv, rows] is the selection table to use
    (the oracle's own, or any other one).  Returns dict(out [n_req, d] fp64,
    lse [n_req], count [n_req] = |A|, mask [n_req, max_k] uint8 if asked).
    """
    cu_q, cu_k, qp = _geom(w, cu_q, cu_k, q_pos0)
    if reqs is None:
        rr, hh = np.meshgrid(np.arange(w.total_q), np.arange(w.h_q), indexing="ij")
        reqs, heads = rr.reshape(-1), hh.reshape(-1)
    reqs, heads = _i64(reqs), _i32(heads)
    idx = _i32(idx)
    n_idx = _i32(n_idx)
    n = len(reqs)
    out = np.empty((n, w.head_dim), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    cnt = np.empty(n, dtype=np.int64)
    stride = max(w.seqlens_k)
    mask = np.empty((n, stride), dtype=np.uint8) if want_mask else None
    if scale is None:
        scale = 1.0 / np.sqrt(w.head_dim)
    rc = lib().or_attend(
        w.batch, w.h_q, w.h_kv, w.head_dim, _ptr(cu_q, _i32p), _ptr(cu_k, _i32p), _ptr(qp, _i32p),
        w.block, w.n_init, w.window, int(w.shared_selection), ctypes.c_double(scale), w.dtype,
        _ptr(q), _ptr(k), _ptr(v), _ptr(idx, _i32p), _ptr(n_idx, _i32p),
        ctypes.c_int64(idx.shape[1]), idx.shape[2], ctypes.c_int64(n), _ptr(reqs, _i64p),
        _ptr(heads, _i32p), _ptr(out, _f64p), _ptr(lse, _f64p), _ptr(cnt, _i64p),
        _ptr(mask, _u8p), ctypes.c_int64(stride))
    assert rc == 0
    return dict(out=out, lse=lse, count=cnt, mask=mask, reqs=reqs, heads=heads)


def run(w, x, rows=None, reqs=None, heads=None):
    """compress -> select (all rows) -> attend (all requests, or the given ones)."""
    kc = compress(w, x["k"]) if w.block > 1 else None
    sel = select(w, x["q"], kc, x["k"])
    idx, n = table(w, sel)
    att = attend(w, x["q"], x["k"], x["v"], idx, n, reqs=reqs, heads=heads)
    return dict(k_cmp=kc, sel=sel, idx=idx, n_idx=n, **att)


def bucket_build(w, k_cmp, cu_k=None) -> dict:
    """The LSA flat bucket index of every complete cluster block, from pooled keys
    ``k_cmp`` [Hkv, batch, nb_max, d] (fp64, from ``compress``): members [Hkv, batch,
    n_cb, C/g] grouped by bucket, offsets [.., NB + 1], centroids [.., NB, d] and the
    smallest relative decision margin of each block (inf when no decision was close)."""
    _, cu_k, _ = _geom(w, None, cu_k, None)
    g, C, NB = w.block, w.bucket_block, w.bucket_count
    M = C // g
    ncb = max(w.seqlens_k) // C
    nb_max = -(-max(w.seqlens_k) // g)
    k_cmp = np.ascontiguousarray(k_cmp, dtype=np.float64)
    member = np.empty((w.h_kv, w.batch, ncb, M), dtype=np.int32)
    offset = np.empty((w.h_kv, w.batch, ncb, NB + 1), dtype=np.int32)
    cent = np.empty((w.h_kv, w.batch, ncb, NB, w.head_dim), dtype=np.float64)
    margin = np.empty((w.h_kv, w.batch, ncb), dtype=np.float64)
    rc = lib().or_bucket_build(w.batch, w.h_kv, w.head_dim, _ptr(cu_k, _i32p), g, C, NB, w.bucket_cap,
                               _ptr(k_cmp, _f64p), ctypes.c_int64(nb_max), ctypes.c_int64(ncb),
                               _ptr(member, _i32p), _ptr(offset, _i32p), _ptr(cent, _f64p), _ptr(margin, _f64p))
    assert rc == 0
    return dict(member=member, offset=offset, centroid=cent, margin=margin)


def bucket_select(w, q_sel, index, rows=None, heads=None, q_pos0=None, cu_q=None, cu_k=None) -> dict:
    """Flat bucket retrieval for (row, KV head) requests: the w.bucket_topk best buckets
    expanded to their member groups outside the sink and window (ascending, -1 padded
    to kb * cap / g).  Returns
    dict(idx, n, nbk (buckets taken), sk / sk1 / floor (bucket-score near-tie data))."""
    cu_q, cu_k, qp = _geom(w, cu_q, cu_k, q_pos0)
    if rows is None:
        rr, hh = np.meshgrid(np.arange(w.rows), np.arange(w.h_kv), indexing="xy")
        heads, rows = hh.reshape(-1), rr.reshape(-1)
    rows, heads = _i64(rows), _i32(heads)
    n = len(rows)
    kcap = max(w.bucket_topk * (w.bucket_cap // w.block), 1)
    idx = np.empty((n, kcap), dtype=np.int32)
    nn, nbk = np.empty(n, dtype=np.int32), np.empty(n, dtype=np.int32)
    sk, sk1, fl = (np.empty(n, dtype=np.float64) for _ in range(3))
    ncb = index["member"].shape[2]
    rc = lib().or_bucket_select(
        w.batch, w.h_q, w.h_kv, w.head_dim, _ptr(cu_q, _i32p), _ptr(cu_k, _i32p), _ptr(qp, _i32p), w.block,
        w.n_init, w.window, w.bucket_block, w.bucket_count, w.bucket_topk, int(w.shared_selection), w.dtype, _ptr(q_sel),
        _ptr(index["member"], _i32p), _ptr(index["offset"], _i32p), _ptr(index["centroid"], _f64p),
        ctypes.c_int64(ncb), ctypes.c_int64(n), _ptr(rows, _i64p), _ptr(heads, _i32p), kcap, _ptr(idx, _i32p),
        _ptr(nn, _i32p), _ptr(sk, _f64p), _ptr(sk1, _f64p), _ptr(fl, _f64p), _ptr(nbk, _i32p))
    assert rc == 0, "expansion exceeded the table width"
    return dict(idx=idx, n=nn, nbk=nbk, sk=sk, sk1=sk1, floor=fl, rows=rows, heads=heads)
