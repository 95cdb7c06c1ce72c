"""sparse_attn_fwd_noalloc through the C ABI (needs an MI355X): the attention call
that allocates nothing, its split partials in the library's fixed device scratch.

Two calls in a row, the second with a smaller input, on shapes where the
attention is split (so the scratch is really written and read): each output and
lse must equal sparse_attn_fwd's on the same inputs bit for bit (the same
kernels and split plan), and also meet the oracle's bars.  An fp32 shape covers
the VALU kernel and its combine, a bf16 decode batch the matrix-core gather.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import top_block_sparse_mean_amd as sa
from workloads import DTYPE_BF16, decode_32k, tiny_fp32_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _case(w):
    x, xg = parity.gen_pair(w)
    p = parity.params_for(w)
    kc = sa.compress(p, xg["k"]) if w.block > 1 else None
    idx, n_idx = sa.select(p, xg["q"], kc, xg["k"])
    torch.cuda.synchronize()
    return x, xg, p, idx, n_idx


def _compare(w, x, xg, p, idx, n_idx):
    fwd_bytes = sa.workspace_size(p)[1]
    assert fwd_bytes > 0, "the shape must split its attention, or the scratch is never used"
    ref, ref_lse = sa.fwd(p, xg["q"], xg["k"], xg["v"], idx, n_idx, want_lse=True)
    out = torch.full_like(xg["q"], float("nan"))
    lse = torch.full((w.h_q, w.total_q), float("nan"), dtype=torch.float32, device="cuda")
    sa.fwd_noalloc(p, xg["q"], xg["k"], xg["v"], idx, n_idx, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32),
                       ref.view(torch.int16 if ref.dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(lse, ref_lse)
    gi, gn = idx.cpu().numpy(), n_idx.cpu().numpy()
    att = oracle.attend(w, x["q"], x["k"], x["v"], gi, gn)
    got = out.float().cpu().reshape(-1, w.head_dim).double().numpy()
    err = np.abs(got - att["out"]).max()
    if w.dtype == DTYPE_BF16:
        assert err / np.abs(att["out"]).max() <= parity.BF16_REL, err
    else:
        assert err <= parity.F32_ABS, err
    return fwd_bytes


@pytest.mark.parametrize("shapes", [
    pytest.param((decode_32k().scaled(seqlens_k=[8192, 6001, 4096 + 5], seqlens_q=[1] * 3),
                  decode_32k().scaled(seqlens_k=[2048 + 17], seqlens_q=[1])), id="bf16_decode"),
    pytest.param((tiny_fp32_prefill().scaled(seqlens_k=[1500, 900], seqlens_q=[40, 9]),
                  tiny_fp32_prefill().scaled(seqlens_k=[700], seqlens_q=[5])), id="fp32_prefill"),
])
def test_noalloc_matches_fwd_twice(shapes):
    big, smaller = shapes
    first = _compare(big, *_case(big))
    second = _compare(smaller, *_case(smaller))
    assert second < first
