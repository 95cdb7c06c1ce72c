"""Selector-driven top-k block-sparse attention for AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI in include/sparse_attn.h.  It only marshals
arguments: every step of the path (pooling, scoring, top-k, attention) runs in
the HIP kernels of libsparse_attn.so.  PyTorch provides device memory and the
current stream.  There is no CPU fallback: if the library is not built, every
call raises.

    p = Params.from_lengths(seqlens_q, seqlens_k, device="cuda", h_q=32, h_kv=8,
                            head_dim=128, block=64, topk=32, n_init=64, window=128,
                            dtype=torch.bfloat16)
    k_cmp = compress(p, k)
    idx, n_idx = select(p, q, k_cmp, k)
    out = fwd(p, q, k, v, idx, n_idx)

A decode loop appends each step's keys and values first (``append_kv``), which also
re-pools the block the new token falls in; ``block_table=`` / ``page_size=`` switch
K and V to a paged cache read through the block table.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._lib import (EXPORTS, LIB_PATH, SA_CHECK_PAGE, SA_CHECK_SEQ, SA_CHECK_TABLE,  # noqa: F401
                   SA_CHECK_TOKEN, SA_DTYPE_BF16, SA_DTYPE_F32, SA_POOL_L2SUM, SA_POOL_MEAN, SA_SELECT_ATTN, SA_SELECT_MAX, SA_SELECT_SOFTMAX, SA_SELECT_SUM, SaBucketIndex,
                   SaParams, SparseAttnError, check, lib)

__all__ = ["Params", "validate", "workspace_size", "compress", "compress_tail", "append_kv", "select",
           "append_select", "fwd", "fwd_noalloc", "decode_step", "BucketIndex", "bucket_build", "bucket_select",
           "abi_version", "SparseAttnError", "SA_POOL_MEAN", "SA_POOL_L2SUM", "SA_SELECT_SUM", "SA_SELECT_SOFTMAX",
           "SA_SELECT_MAX", "SA_SELECT_ATTN", "LIB_PATH", "EXPORTS", "check_flags", "SA_CHECK_SEQ",
           "SA_CHECK_TABLE", "SA_CHECK_PAGE", "SA_CHECK_TOKEN"]

_DT = {torch.float32: SA_DTYPE_F32, torch.bfloat16: SA_DTYPE_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class Params:
    """One call configuration (sa_params); holds the device tensors it points at."""

    def __init__(self, *, batch: int, h_q: int, h_kv: int, head_dim: int, cu_seqlens_q: torch.Tensor,
                 cu_seqlens_k: torch.Tensor, max_q: int, max_k: int, total_q: int, total_k: int,
                 block: int, topk: int, n_init: int, window: int, dtype=torch.bfloat16,
                 pool: int = SA_POOL_MEAN, shared_selection: int = 0,
                 topk_per_seq: Optional[torch.Tensor] = None, q_pos0: Optional[torch.Tensor] = None,
                 softmax_scale: float = 0.0, block_table: Optional[torch.Tensor] = None, page_size: int = 0,
                 pool_overlap: int = 0, select_mode: int = SA_SELECT_SUM, select_tau: float = 0.0):
        """block_table: int32 [batch, max_pages] page ids of a paged K/V cache (K and V
        arguments are then page pools [pages * page_size, h_kv, d]); None = packed K/V.
        pool_overlap / select_mode / select_tau: the selector variants (overlapping pooling
        windows; the group score as a sum of per-head softmaxes at temperature tau, or as
        the max over heads)."""
        self._keep = (cu_seqlens_q, cu_seqlens_k, topk_per_seq, q_pos0, block_table)
        self.dtype = dtype
        s = SaParams()
        s.batch, s.h_q, s.h_kv, s.head_dim = batch, h_q, h_kv, head_dim
        s.max_q, s.max_k, s.total_q, s.total_k = max_q, max_k, total_q, total_k
        s.cu_seqlens_q = cu_seqlens_q.data_ptr()
        s.cu_seqlens_k = cu_seqlens_k.data_ptr()
        s.q_pos0 = None if q_pos0 is None else q_pos0.data_ptr()
        s.block, s.pool, s.topk = block, pool, topk
        s.topk_per_seq = None if topk_per_seq is None else topk_per_seq.data_ptr()
        s.n_init, s.window, s.shared_selection = n_init, window, shared_selection
        s.softmax_scale = softmax_scale
        s.dtype = _DT[dtype]
        s.pool_overlap, s.select_mode, s.select_temperature = pool_overlap, select_mode, select_tau
        if block_table is not None:
            if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
                raise ValueError("block_table must be a contiguous int32 [batch, max_pages] tensor")
            s.block_table = block_table.data_ptr()
            s.max_pages = block_table.shape[1]
            s.page_size = page_size
        self.s = s

    @classmethod
    def from_lengths(cls, seqlens_q: Sequence[int], seqlens_k: Sequence[int], device="cuda",
                     topk_per_seq: Optional[Sequence[int]] = None, q_pos0: Optional[Sequence[int]] = None,
                     block_table=None, **kw) -> "Params":
        def cu(lens):
            out = [0]
            for x in lens:
                out.append(out[-1] + int(x))
            return torch.tensor(out, dtype=torch.int32, device=device)

        tps = None if topk_per_seq is None else torch.tensor(list(topk_per_seq), dtype=torch.int32,
                                                             device=device)
        qp = None if q_pos0 is None else torch.tensor(list(q_pos0), dtype=torch.int32, device=device)
        if block_table is not None and not isinstance(block_table, torch.Tensor):
            block_table = torch.tensor(block_table, dtype=torch.int32, device=device)
        return cls(batch=len(seqlens_k), cu_seqlens_q=cu(seqlens_q), cu_seqlens_k=cu(seqlens_k),
                   max_q=max(seqlens_q), max_k=max(seqlens_k), total_q=sum(seqlens_q),
                   total_k=sum(seqlens_k), topk_per_seq=tps, q_pos0=qp, block_table=block_table, **kw)

    @property
    def rows(self) -> int:
        return self.s.batch if self.s.shared_selection else self.s.total_q

    @property
    def nb_max(self) -> int:
        return -(-self.s.max_k // self.s.block)

    def ref(self):
        return ctypes.byref(self.s)


def abi_version() -> int:
    return lib().sparse_attn_abi_version()


def check_flags(clear: bool = True) -> int:
    """The contract-check bits the checked library has set on the current GPU since they
    were last cleared (SA_CHECK_*); clears them unless clear is False.  Synchronise the
    streams that ran the checked work first.  Raises in a library built without checks."""
    v = ctypes.c_uint32(0)
    check("sparse_attn_check_flags", lib().sparse_attn_check_flags(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


def validate(p: Params) -> None:
    check("sparse_attn_validate", lib().sparse_attn_validate(p.ref()))


def workspace_size(p: Params):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    check("sparse_attn_workspace_size", lib().sparse_attn_workspace_size(p.ref(), ctypes.byref(a),
                                                                         ctypes.byref(b)))
    return a.value, b.value


def _ws(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def compress(p: Params, k: torch.Tensor, k_cmp: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if k_cmp is None:
        k_cmp = torch.empty((p.s.h_kv, p.s.batch, p.nb_max, p.s.head_dim), dtype=torch.float32,
                            device=k.device)
    check("sparse_attn_compress", lib().sparse_attn_compress(p.ref(), _ptr(k), _ptr(k_cmp), _stream(stream)))
    return k_cmp


def compress_tail(p: Params, n_tail_blocks: int, k: torch.Tensor, k_cmp: torch.Tensor, stream=None) -> torch.Tensor:
    check("sparse_attn_compress_tail", lib().sparse_attn_compress_tail(p.ref(), int(n_tail_blocks), _ptr(k),
                                                                       _ptr(k_cmp), _stream(stream)))
    return k_cmp


def append_kv(p: Params, k_new: torch.Tensor, v_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              k_cmp: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write the new tokens' keys and values (one row per query row of ``p``) into the
    cache and re-pool the blocks they fall in (k_cmp, when given)."""
    check("sparse_attn_append_kv", lib().sparse_attn_append_kv(p.ref(), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v),
                                                               _ptr(k_cmp), _stream(stream)))


def _set_events(p: Params, events) -> None:
    """The params' timing event pair: torch.cuda.Event objects (recorded once, so their
    handles exist) or raw hipEvent_t handles as ints; None clears it."""
    for i in range(2):
        e = None if events is None else events[i]
        p.s.timing_events[i] = e if e is None or isinstance(e, int) else e.cuda_event


def select(p: Params, q_sel: torch.Tensor, k_cmp: Optional[torch.Tensor], k: Optional[torch.Tensor],
           idx: Optional[torch.Tensor] = None, n_idx: Optional[torch.Tensor] = None,
           ws: Optional[torch.Tensor] = None, stream=None, attn_lse: Optional[torch.Tensor] = None,
           events=None, boundary: Optional[torch.Tensor] = None, want_boundary: bool = False):
    """Top-k selection.  With select_mode SA_SELECT_ATTN, q_sel are the verify queries and
    ``attn_lse`` [h_q, total_q] the log-sum-exp their dense attention pass returned.
    ``events`` = (begin, end) pair recorded around the scoring kernel, as for fwd.
    With ``want_boundary`` (or a ``boundary`` tensor [h_kv, rows, 2] fp32) the call also
    returns each row's need-th and (need+1)-th scores: (idx, n_idx, boundary)."""
    dev = q_sel.device
    if idx is None:
        idx = torch.empty((p.s.h_kv, p.rows, max(p.s.topk, 1)), dtype=torch.int32, device=dev)
    if n_idx is None:
        n_idx = torch.empty((p.s.h_kv, p.rows), dtype=torch.int32, device=dev)
    if want_boundary and boundary is None:
        boundary = torch.empty((p.s.h_kv, p.rows, 2), dtype=torch.float32, device=dev)
    ws, nbytes = _ws(workspace_size(p)[0], dev, ws)
    p.s.attn_lse = None if attn_lse is None else attn_lse.data_ptr()
    _set_events(p, events)
    try:
        st = lib().sparse_attn_select(p.ref(), _ptr(q_sel), _ptr(k_cmp), _ptr(k), _ptr(idx), _ptr(n_idx),
                                      _ptr(boundary), _ptr(ws), nbytes, _stream(stream))
    finally:
        p.s.attn_lse = None
        _set_events(p, None)
    check("sparse_attn_select", st)
    return (idx, n_idx, boundary) if boundary is not None else (idx, n_idx)


def append_select(p: Params, k_new: torch.Tensor, v_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  k_cmp: Optional[torch.Tensor], q_sel: torch.Tensor, idx: Optional[torch.Tensor] = None,
                  n_idx: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None, events=None):
    """append_kv then select, in one launch for decode rows (``events`` as for select)."""
    dev = q_sel.device
    if idx is None:
        idx = torch.empty((p.s.h_kv, p.rows, max(p.s.topk, 1)), dtype=torch.int32, device=dev)
    if n_idx is None:
        n_idx = torch.empty((p.s.h_kv, p.rows), dtype=torch.int32, device=dev)
    ws, nbytes = _ws(workspace_size(p)[0], dev, ws)
    _set_events(p, events)
    try:
        st = lib().sparse_attn_append_select(p.ref(), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v), _ptr(k_cmp),
                                             _ptr(q_sel), _ptr(idx), _ptr(n_idx), _ptr(ws), nbytes, _stream(stream))
    finally:
        _set_events(p, None)
    check("sparse_attn_append_select", st)
    return idx, n_idx


def fwd(p: Params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, n_idx: torch.Tensor,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = False,
        ws: Optional[torch.Tensor] = None, stream=None, events=None):
    """Sparse attention; ``events`` = (begin, end) pair recorded around the main attention
    kernel: torch.cuda.Event objects (recorded once, so their handles exist) or raw
    hipEvent_t handles as ints."""
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((p.s.h_q, p.s.total_q), dtype=torch.float32, device=q.device)
    ws, nbytes = _ws(workspace_size(p)[1], q.device, ws)
    _set_events(p, events)
    try:
        st = lib().sparse_attn_fwd(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_idx), _ptr(out),
                                   _ptr(lse), _ptr(ws), nbytes, _stream(stream))
    finally:
        _set_events(p, None)
    check("sparse_attn_fwd", st)
    return (out, lse) if want_lse else out


def decode_step(p: Params, k_new: torch.Tensor, v_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                k_cmp: Optional[torch.Tensor], q: torch.Tensor, idx: Optional[torch.Tensor] = None,
                n_idx: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = False, ws: Optional[torch.Tensor] = None,
                stream=None, events=None):
    """append_kv, select (q as the selector query) and fwd of one decode step, in one launch
    where the step fits it.  Returns (out, idx, n_idx) or, with want_lse, (out, lse, idx, n_idx)."""
    dev = q.device
    if idx is None:
        idx = torch.empty((p.s.h_kv, p.rows, max(p.s.topk, 1)), dtype=torch.int32, device=dev)
    if n_idx is None:
        n_idx = torch.empty((p.s.h_kv, p.rows), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((p.s.h_q, p.s.total_q), dtype=torch.float32, device=dev)
    sel_b, fwd_b = workspace_size(p)
    ws, nbytes = _ws(max(sel_b, fwd_b), dev, ws)
    _set_events(p, events)
    try:
        st = lib().sparse_attn_decode_step(p.ref(), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v), _ptr(k_cmp),
                                           _ptr(q), _ptr(idx), _ptr(n_idx), _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                           _stream(stream))
    finally:
        _set_events(p, None)
    check("sparse_attn_decode_step", st)
    return (out, lse, idx, n_idx) if want_lse else (out, idx, n_idx)


def fwd_noalloc(p: Params, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                n_idx: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """fwd with every buffer supplied by the caller and the split partials in the library's
    fixed device scratch: allocates nothing (for callers that cannot allocate)."""
    st = lib().sparse_attn_fwd_noalloc(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_idx), _ptr(out),
                                       _ptr(lse), _stream(stream))
    check("sparse_attn_fwd_noalloc", st)
    return out


class BucketIndex:
    """Device arrays of an LSA flat bucket index (sa_bucket_index): cluster blocks of
    ``block_tokens`` tokens, ``count`` buckets each, at most ``cap_tokens`` per bucket."""

    def __init__(self, p: Params, block_tokens: int = 512, count: int = 64, cap_tokens: int = 16, device="cuda"):
        s = p.s
        self.blocks_max = max(s.max_k // block_tokens, 1)
        m = block_tokens // s.block
        self.centroid = torch.empty((s.h_kv, s.batch, self.blocks_max, count, s.head_dim), dtype=torch.float32,
                                    device=device)
        self.member = torch.empty((s.h_kv, s.batch, self.blocks_max, m), dtype=torch.int32, device=device)
        self.offset = torch.empty((s.h_kv, s.batch, self.blocks_max, count + 1), dtype=torch.int32, device=device)
        b = SaBucketIndex()
        b.block_tokens, b.count, b.cap_tokens, b.blocks_max = block_tokens, count, cap_tokens, self.blocks_max
        b.centroid, b.member, b.offset = self.centroid.data_ptr(), self.member.data_ptr(), self.offset.data_ptr()
        self.s = b

    def ref(self):
        return ctypes.byref(self.s)


def bucket_build(p: Params, k_cmp: torch.Tensor, index: BucketIndex, stream=None, build_from: int = 0) -> BucketIndex:
    """Cluster the pooled keys of every complete cluster block from ``build_from`` on into buckets
    (earlier blocks are left as they are)."""
    index.s.build_from = int(build_from)
    check("sparse_attn_bucket_build", lib().sparse_attn_bucket_build(p.ref(), _ptr(k_cmp), index.ref(),
                                                                     _stream(stream)))
    return index


def bucket_select(p: Params, q_sel: torch.Tensor, index: BucketIndex, n_buckets: int,
                  idx: Optional[torch.Tensor] = None, n_idx: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None):
    """Flat bucket retrieval; the table width is p's topk (>= n_buckets * cap / block)."""
    dev = q_sel.device
    if idx is None:
        idx = torch.empty((p.s.h_kv, p.rows, p.s.topk), dtype=torch.int32, device=dev)
    if n_idx is None:
        n_idx = torch.empty((p.s.h_kv, p.rows), dtype=torch.int32, device=dev)
    nb = ctypes.c_size_t(0)
    check("sparse_attn_bucket_workspace_size",
          lib().sparse_attn_bucket_workspace_size(p.ref(), index.ref(), int(n_buckets), ctypes.byref(nb)))
    ws, nbytes = _ws(nb.value, dev, ws)
    check("sparse_attn_bucket_select",
          lib().sparse_attn_bucket_select(p.ref(), _ptr(q_sel), index.ref(), int(n_buckets), _ptr(idx), _ptr(n_idx),
                                          _ptr(ws), nbytes, _stream(stream)))
    return idx, n_idx
