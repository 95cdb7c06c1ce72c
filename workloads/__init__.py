"""Seeded synthetic workloads (geometry + input generators) shared by the tests,
the benchmark and the oracle checks.  No part of the method is computed here."""
from .configs import (DTYPE_BF16, DTYPE_F32, FULL, POOL_L2SUM, POOL_MEAN, SELECT_ATTN, SELECT_MAX,  # noqa: F401
                      SELECT_SOFTMAX, SELECT_SUM, Workload,
                      chunked_prefill_1m, decode_32k, draft_decode, draft_keep, prefill_128k,
                      small, tiny_fp32_prefill)
from .gen import cu_seqlens, generate, hot_blocks, needle_groups  # noqa: F401
from .paging import PageLayout, from_pages, page_layout, to_pages, token_rows  # noqa: F401
