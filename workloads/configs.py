"""The five synthetic workloads of selector-driven top-k sparse attention, plus
small variants of the same shape family that the CPU oracle finishes in seconds.

A workload fixes the geometry (batch, heads, head size, per-sequence key and
query counts), the selector (pool size g, pooling mode, top-k, sink and window)
and the input structure the generator plants.  It holds none of the method's
arithmetic.

Where the numbers come from:
  * tiny fp32 prefill, decode, long prefill: the block-selection setting of the
    SparDA summary (Method: init tokens + sliding window + top-k blocks over
    mean-pooled keys), at the sizes of its 32K decode / 128K prefill runs
    (Experiments).
  * draft decode: the S3R review (sparse drafting: recent window + top-K by
    score, budget clamped between Kmin and s*|C|, k = 6 drafts sharing one
    selection).
  * 1M chunked prefill: the LSA deep-read (§2.2 L2-normalise and sum 4 keys;
    §2.3 four sink keys, a 512-key window and 2048 long-range keys).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

POOL_MEAN = 0
POOL_L2SUM = 1

# how a GQA group's heads combine into one block score
SELECT_SUM = 0        # the heads' queries summed into one selector query
SELECT_SOFTMAX = 1    # sum over heads of each head's softmax over the candidates (temperature tau)
SELECT_MAX = 2        # max over heads of the per-head score
SELECT_ATTN = 3       # attention mass of a dense verify pass (every query and head of the row)

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass
class Workload:
    name: str
    dtype: int                 # DTYPE_F32 / DTYPE_BF16 for Q, K, V, O
    h_q: int
    h_kv: int
    head_dim: int
    seqlens_k: List[int]       # N_b, keys per sequence
    seqlens_q: List[int]       # M_b, queries per sequence (right-aligned)
    block: int                 # g
    pool: int
    topk: int                  # k (blocks; tokens when g == 1); capacity when topk_per_seq is set
    n_init: int
    window: int
    shared_selection: int = 0  # 1: one selection per sequence, shared by its queries
    topk_per_seq: Optional[List[int]] = None
    pool_overlap: int = 0      # o: each block's pooling window reaches o tokens back (kernel g + o, stride g)
    select_mode: int = SELECT_SUM
    select_tau: float = 0.0    # softmax temperature of SELECT_SOFTMAX; 0 = sqrt(d)
    # LSA flat bucket index: cluster blocks of bucket_block tokens, bucket_count buckets each,
    # at most bucket_cap tokens per bucket; retrieval takes the bucket_topk best buckets
    bucket_block: int = 512
    bucket_count: int = 64
    bucket_cap: int = 16
    bucket_topk: int = 256
    structure: str = "iid"     # iid | hot_blocks | lowrank | needles
    seed: int = 0
    # structure knobs
    n_hot: int = 8
    hot_shift: float = 2.0
    lowrank_rank: int = 8
    lowrank_scale: float = 0.5
    n_needles: int = 64
    needle_shift: float = 2.0
    needle_segment: int = 64

    @property
    def batch(self) -> int:
        return len(self.seqlens_k)

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def total_k(self) -> int:
        return sum(self.seqlens_k)

    @property
    def total_q(self) -> int:
        return sum(self.seqlens_q)

    @property
    def max_k(self) -> int:
        return max(self.seqlens_k)

    @property
    def max_q(self) -> int:
        return max(self.seqlens_q)

    @property
    def rows(self) -> int:
        """Selection rows per KV head: one per query, or one per sequence."""
        return self.batch if self.shared_selection else self.total_q

    @property
    def nb_max(self) -> int:
        return -(-self.max_k // self.block)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _lognormal_lengths(n: int, median: int, sigma: float, lo: int, hi: int, seed: int) -> List[int]:
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal(n)
    return [int(min(max(round(median * math.exp(sigma * float(x))), lo), hi)) for x in z]


def draft_keep(t_hist: int, kmin: int = 256, frac: float = 0.1) -> int:
    """S3R budget clamp as read here: keep = max(Kmin, floor(s * T))."""
    return max(kmin, int(math.floor(frac * t_hist)))


def tiny_fp32_prefill() -> Workload:
    return Workload(name="tiny_fp32_prefill", dtype=DTYPE_F32, h_q=4, h_kv=1, head_dim=64,
                    seqlens_k=[2048], seqlens_q=[2048], block=64, pool=POOL_MEAN, topk=4,
                    n_init=64, window=128, structure="iid", seed=1001)


def decode_32k(batch: int = 32, t: int = 32768) -> Workload:
    return Workload(name="bf16_decode_32k", dtype=DTYPE_BF16, h_q=32, h_kv=8, head_dim=128,
                    seqlens_k=[t] * batch, seqlens_q=[1] * batch, block=64, pool=POOL_MEAN,
                    topk=32, n_init=64, window=128, structure="hot_blocks", seed=1002)


def prefill_128k(t: int = 131072) -> Workload:
    return Workload(name="bf16_prefill_128k", dtype=DTYPE_BF16, h_q=32, h_kv=8, head_dim=128,
                    seqlens_k=[t], seqlens_q=[t], block=64, pool=POOL_MEAN, topk=64,
                    n_init=64, window=512, structure="lowrank", seed=1003)


def draft_decode(batch: int = 64, median: int = 4096, lo: int = 512, hi: int = 32768,
                 n_draft: int = 6, window: int = 64, seed: int = 1004) -> Workload:
    hist = _lognormal_lengths(batch, median, 1.0, lo, hi, seed)
    keep = [draft_keep(t) for t in hist]
    topk = [kp - window for kp in keep]
    return Workload(name="bf16_draft_decode", dtype=DTYPE_BF16, h_q=16, h_kv=8, head_dim=128,
                    seqlens_k=[t + n_draft for t in hist], seqlens_q=[n_draft] * batch,
                    block=1, pool=POOL_MEAN, topk=max(topk), topk_per_seq=topk,
                    n_init=0, window=window, shared_selection=1, structure="iid", seed=seed)


def chunked_prefill_1m(t: int = 1048576, chunk: int = 4096) -> Workload:
    return Workload(name="bf16_chunked_prefill_1m", dtype=DTYPE_BF16, h_q=16, h_kv=1,
                    head_dim=128, seqlens_k=[t], seqlens_q=[chunk], block=4, pool=POOL_L2SUM,
                    topk=512, n_init=4, window=512, structure="needles", seed=1005)


FULL = {
    "tiny_fp32_prefill": tiny_fp32_prefill,
    "bf16_decode_32k": decode_32k,
    "bf16_prefill_128k": prefill_128k,
    "bf16_draft_decode": draft_decode,
    "bf16_chunked_prefill_1m": chunked_prefill_1m,
}


def small(name: str) -> Workload:
    """Same shape family at a size the oracle finishes in seconds; ragged tails on purpose."""
    if name == "tiny_fp32_prefill":
        return tiny_fp32_prefill().scaled(seqlens_k=[1000, 2048 + 37], seqlens_q=[1000, 700],
                                          name="tiny_fp32_prefill_small")
    if name == "bf16_decode_32k":
        return decode_32k().scaled(seqlens_k=[4096, 3001, 2113 + 64, 777, 130], seqlens_q=[1] * 5,
                                   name="bf16_decode_small")
    if name == "bf16_prefill_128k":
        return prefill_128k().scaled(seqlens_k=[3000 + 29], seqlens_q=[3000 + 29], topk=16,
                                     name="bf16_prefill_small")
    if name == "bf16_draft_decode":
        return draft_decode(batch=6, median=700, lo=320, hi=3000).scaled(name="bf16_draft_small")
    if name == "bf16_chunked_prefill_1m":
        return chunked_prefill_1m().scaled(seqlens_k=[16384 + 3], seqlens_q=[300], topk=64,
                                           n_needles=4, name="bf16_chunked_small")
    raise KeyError(name)
