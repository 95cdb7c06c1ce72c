"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every
symbol include/sparse_attn.h declares, and rejects bad arguments with the
documented status before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

import top_block_sparse_mean_amd as sa
from top_block_sparse_mean_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

INVALID, UNSUPPORTED, WORKSPACE = _lib.SA_ERR_INVALID_ARG, _lib.SA_ERR_UNSUPPORTED, _lib.SA_ERR_WORKSPACE
FAKE = 1 << 20          # a 16-byte aligned stand-in device address: never dereferenced by host checks


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sparse_attn_[a-z_]+)\s*\(", text)))


def params(**kw):
    s = _lib.SaParams()
    base = dict(batch=2, h_q=8, h_kv=2, head_dim=128, max_q=1, max_k=4096, total_q=2, total_k=8192,
                cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, q_pos0=None, block=64, pool=0, topk=8,
                topk_per_seq=None, n_init=64, window=128, shared_selection=0, softmax_scale=0.0, dtype=1)
    base.update(kw)
    for k, v in base.items():
        setattr(s, k, v)
    return s


def status(fn, *args):
    return getattr(_lib.lib(), fn)(*args)


def test_library_loads_and_version():
    assert _lib.lib() is not None
    assert sa.abi_version() == 10


def test_struct_layout_matches_header(tmp_path):
    """The ctypes view of sa_params has the C struct's size and field offsets."""
    fields = [f for f, _ in _lib.SaParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sparse_attn.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(sa_params));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(sa_params, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(_lib.SaParams)
    assert got[1:] == [getattr(_lib.SaParams, f).offset for f in fields]


def test_every_declared_symbol_is_exported():
    decl = declared_symbols()
    assert set(decl) == set(_lib.EXPORTS), decl
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sparse_attn_\w+)", out))
    missing = [s for s in decl if s not in exported]
    assert not missing, missing
    for s in decl:
        assert hasattr(_lib.lib(), s)


def test_checked_build_exports_the_same_symbols():
    """The debugging build with contract checks is a drop-in replacement."""
    from top_block_sparse_mean_amd import build
    assert os.path.exists(build.CHECKED_OUT), "libsparse_attn_checked.so is not built"
    out = subprocess.run(["nm", "-D", "--defined-only", build.CHECKED_OUT], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sparse_attn_\w+)", out))
    assert set(declared_symbols()) <= exported


def test_check_flags_without_checks():
    """The plain build carries no contract checks: the call says so (flags zeroed) and
    touches no device; a NULL output is rejected first."""
    v = ctypes.c_uint32(7)
    if _lib.LIB_PATH.endswith("libsparse_attn_checked.so"):
        pytest.skip("the checked build is loaded")
    assert status("sparse_attn_check_flags", ctypes.byref(v), 1) == UNSUPPORTED
    assert v.value == 0
    assert "without contract checks" in _lib.lib().sparse_attn_last_error().decode()
    assert status("sparse_attn_check_flags", None, 1) == INVALID
    assert "NULL" in _lib.lib().sparse_attn_last_error().decode()
    with pytest.raises(sa.SparseAttnError):
        sa.check_flags()


def test_every_export_has_a_c_signature():
    """Each entry point's argument types are declared to ctypes: without them Python ints
    travel as 32-bit C ints, and a size_t argument such as a workspace size would carry
    whatever the upper half of its register held."""
    L = _lib.lib()
    assert [n for n in _lib.EXPORTS if getattr(L, n).argtypes is None] == []


def test_status_strings():
    L = _lib.lib()
    names = [L.sparse_attn_status_string(i).decode() for i in range(5)]
    assert names[0] == "ok" and len(set(names)) == 5
    assert L.sparse_attn_status_string(99)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, INVALID), ("h_q", 7, INVALID), ("h_kv", 0, INVALID), ("head_dim", 96, UNSUPPORTED),
    ("max_q", 0, INVALID), ("max_k", 0, INVALID), ("total_k", 0, INVALID), ("total_q", 0, INVALID), ("cu_seqlens_q", None, INVALID),
    ("cu_seqlens_k", None, INVALID), ("block", 0, INVALID), ("pool", 7, INVALID), ("topk", -1, INVALID), ("topk", (1 << 24) + 1, UNSUPPORTED),
    ("n_init", -2, INVALID), ("window", 0, INVALID), ("shared_selection", 2, INVALID), ("dtype", 5, INVALID),
    ("softmax_scale", -1.0, INVALID), ("softmax_scale", float("inf"), INVALID),
    ("pool_overlap", -1, INVALID), ("pool_overlap", (1 << 20) + 1, INVALID),
    ("select_mode", -1, INVALID), ("select_mode", 4, INVALID), ("select_temperature", -0.5, INVALID),
    ("select_temperature", float("inf"), INVALID),
    ("h_q", 2 * 65, UNSUPPORTED)])
def test_validate_rejects(field, value, code):
    p = params(**{field: value})
    if field == "h_q" and value == 130:
        p.h_kv = 2
    assert status("sparse_attn_validate", ctypes.byref(p)) == code
    msg = _lib.lib().sparse_attn_last_error().decode()
    assert msg


@pytest.mark.parametrize("page_size,max_pages", [(0, 64), (3, 64), (1 << 21, 64), (64, 63), (-64, 64)])
def test_validate_rejects_bad_paging(page_size, max_pages):
    p = params(block_table=FAKE, page_size=page_size, max_pages=max_pages)   # max_k 4096
    assert status("sparse_attn_validate", ctypes.byref(p)) == INVALID
    assert "page" in _lib.lib().sparse_attn_last_error().decode()


def test_validate_accepts_paging():
    for ps, mp in [(1, 4096), (16, 256), (64, 64), (4096, 1), (1 << 20, 1)]:
        assert status("sparse_attn_validate", ctypes.byref(params(block_table=FAKE, page_size=ps,
                                                                  max_pages=mp))) == 0
    # without a block table the paging fields are ignored
    assert status("sparse_attn_validate", ctypes.byref(params(page_size=3, max_pages=0))) == 0


def test_validate_accepts_and_clears_error():
    assert status("sparse_attn_validate", None) == INVALID
    assert status("sparse_attn_validate", ctypes.byref(params())) == 0
    assert _lib.lib().sparse_attn_last_error().decode() == ""


def _ws(p):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert status("sparse_attn_workspace_size", ctypes.byref(p), ctypes.byref(a), ctypes.byref(b)) == 0
    return a.value, b.value


def test_workspace_sizes():
    # decode shape: (key, position) survivors of each 128-candidate part of every (row, KV
    # head), min(k + 1, 128) per part; one attention split per (query, KV head) unit when
    # there are enough units, else partials for the combine
    sel, fwd = _ws(params())
    assert sel == 2 * 2 * 1 * 9 * 8 and fwd > 0 and fwd % (130 * 4) == 0
    assert _ws(params(batch=64, total_q=64, max_k=4096, total_k=64 * 4096))[0] == 2 * 64 * 1 * 9 * 8
    # rows x KV heads >= 256: one workgroup per (row, KV head) selects from LDS, no workspace
    assert _ws(params(batch=128, total_q=128, max_k=4096, total_k=128 * 4096)) == (0, 0)
    assert _ws(params(max_k=32768, total_k=65536, topk=32))[0] == 2 * 2 * 4 * 33 * 8
    # prefill: scores of every (row, block) are kept, rows padded to a multiple of 32 plus
    # 32 (the first candidate's group starts a 128-byte line): h_kv * rows * (64 + 32) * 4
    p = params(batch=1, max_q=4096, total_q=4096, max_k=4096, total_k=4096)
    sel, fwd = _ws(p)
    assert sel == 2 * 4096 * 96 * 4
    # long prefill rows (> 2048 candidates): the scores plus each row's maxima of every
    # 32 candidates (row stride rounded up to a multiple of 4)
    p = params(batch=1, max_q=512, total_q=512, max_k=65536, total_k=65536, block=4)
    assert _ws(p)[0] == 2 * 512 * (16384 + 32 + 512) * 4
    p = params(batch=1, max_q=512, total_q=512, max_k=65536 + 4 * 33, total_k=65536 + 4 * 33, block=4)
    assert _ws(p)[0] == 2 * 512 * (16384 + 64 + 32 + 516) * 4
    # token-level shared selection with long rows: scores in the workspace
    p = params(block=1, shared_selection=1, max_q=6, total_q=12, max_k=20000, total_k=40000, topk=3000)
    sel, _ = _ws(p)
    assert sel == 2 * 2 * (20000 + 32) * 4
    # k = 0: nothing to score
    assert _ws(params(topk=0))[0] == 0
    # per-head group scores: order keys of every (row, block); SOFTMAX also keeps every head's logit
    assert _ws(params(select_mode=2))[0] == 2 * 2 * 96 * 4
    assert _ws(params(select_mode=1))[0] == 2 * 2 * 96 * 4 * (1 + 4)


def test_long_attended_sets_leave_the_gather_kernel():
    """The bf16 gather kernel lists each split's tokens in LDS (8192 per split, at most 64
    splits merged by the combine); a set longer than 64 * 8192 tokens must go to the VALU
    kernel, which walks positions with no list (at most 32 splits). Checked through the
    attention workspace each plan asks for; nothing runs on a device."""
    part = 8 * 130 * 4                      # one split's partials of the query's 8 heads, d = 128
    at_cap = params(batch=1, max_q=1, total_q=1, max_k=1 << 19, total_k=1 << 19, topk=8192)
    assert _ws(at_cap)[1] == 64 * part       # 524288 tokens: gather kernel, 64 splits of 8192
    beyond = params(batch=1, max_q=1, total_q=1, max_k=1 << 20, total_k=1 << 20, topk=16384)
    assert _ws(beyond)[1] == 32 * part       # 1048576 tokens: VALU kernel
    drafts = params(batch=1, max_q=6, total_q=6, max_k=(1 << 20) + 6, total_k=(1 << 20) + 6, block=1,
                    topk=1 << 20, shared_selection=1, h_q=4)
    assert _ws(drafts)[1] == 6 * 4 * 32 * 130 * 4


def test_fwd_noalloc_rejects_partials_above_its_scratch():
    """The no-allocation attention keeps split partials in a fixed 32 MiB device array: a
    decode batch whose 524288-token sets need 64 splits (34 MB of partials) is refused on
    the host with SA_ERR_WORKSPACE before any HIP call; a missing pointer is refused too."""
    vp = ctypes.c_void_p
    big = params(batch=32, h_q=32, h_kv=8, max_q=1, total_q=32, max_k=1 << 19, total_k=32 << 19, topk=8192)
    assert _ws(big)[1] == 32 * 32 * 64 * 130 * 4 > 32 << 20
    args = [vp(FAKE)] * 6 + [None, None]
    assert status("sparse_attn_fwd_noalloc", ctypes.byref(big), *args) == WORKSPACE
    assert b"32" in _lib.lib().sparse_attn_last_error()
    assert status("sparse_attn_fwd_noalloc", ctypes.byref(params()), None, *args[1:]) == INVALID


def test_append_select_rejects_bad_arguments():
    vp = ctypes.c_void_p
    ok = [vp(FAKE)] * 5
    p = ctypes.byref(params())
    # k_new missing; then q_sel missing; then a misaligned k_cmp
    assert status("sparse_attn_append_select", p, None, *ok[:4], vp(FAKE), vp(FAKE), vp(FAKE), None, 0, None) == INVALID
    assert status("sparse_attn_append_select", p, *ok, None, vp(FAKE), vp(FAKE), None, 0, None) == INVALID
    assert status("sparse_attn_append_select", p, *ok[:4], vp(FAKE + 4), vp(FAKE), vp(FAKE), vp(FAKE), None, 0,
                  None) == INVALID
    # the verify-pass score needs sparse_attn_select
    pa = params(select_mode=3)
    pa.attn_lse = FAKE
    assert status("sparse_attn_append_select", ctypes.byref(pa), *ok, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1 << 30,
                  None) == INVALID
    assert "SA_SELECT_ATTN" in _lib.lib().sparse_attn_last_error().decode()
    # decode rows need no select workspace once rows x KV heads fill the GPU; small batches do
    assert status("sparse_attn_append_select", p, *ok, vp(FAKE), vp(FAKE), vp(FAKE), None, 0, None) == WORKSPACE


def test_calls_reject_null_and_misaligned_pointers():
    p = ctypes.byref(params())
    vp = ctypes.c_void_p
    assert status("sparse_attn_compress", p, None, vp(FAKE), None) == INVALID
    assert status("sparse_attn_compress", p, vp(FAKE + 2), vp(FAKE), None) == INVALID
    assert status("sparse_attn_compress_tail", p, 0, vp(FAKE), vp(FAKE), None) == INVALID
    assert status("sparse_attn_select", p, None, vp(FAKE), None, vp(FAKE), vp(FAKE), None, None, 0, None) == INVALID
    assert status("sparse_attn_select", p, vp(FAKE), None, None, vp(FAKE), vp(FAKE), None, None, 0,
                  None) == INVALID
    # the boundary-score output is optional but must hold aligned fp32
    pb = ctypes.byref(params(batch=128, total_q=128))      # row plan: no workspace needed
    assert status("sparse_attn_select", pb, vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), vp(FAKE + 2), None, 0,
                  None) == INVALID
    assert "boundary_scores" in _lib.lib().sparse_attn_last_error().decode()
    assert status("sparse_attn_fwd", p, vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), vp(FAKE), None, None, 0,
                  None) == INVALID
    assert status("sparse_attn_fwd", p, vp(FAKE + 8), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None,
                  None, 0, None) == INVALID
    # append: k_new, v_new, k and v are required; k_cmp is optional but must be aligned
    assert status("sparse_attn_append_kv", p, None, vp(FAKE), vp(FAKE), vp(FAKE), None, None) == INVALID
    assert status("sparse_attn_append_kv", p, vp(FAKE), vp(FAKE), vp(FAKE), None, None, None) == INVALID
    assert status("sparse_attn_append_kv", p, vp(FAKE), vp(FAKE + 2), vp(FAKE), vp(FAKE), None, None) == INVALID
    assert status("sparse_attn_append_kv", p, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE + 4),
                  None) == INVALID
    # attention-mass selection: raw keys and the verify pass's lse are required; rows of
    # more than 64 (query, head) pairs are not built
    pa = ctypes.byref(params(select_mode=3))
    ws = vp(FAKE)
    assert status("sparse_attn_select", pa, vp(FAKE), None, vp(FAKE), vp(FAKE), vp(FAKE), None, ws, 1 << 30,
                  None) == INVALID
    assert "attn_lse" in _lib.lib().sparse_attn_last_error().decode()
    assert status("sparse_attn_select", pa, vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), None, ws, 1 << 30,
                  None) == INVALID
    assert "raw keys" in _lib.lib().sparse_attn_last_error().decode()
    big = params(select_mode=3, shared_selection=1, max_q=20, total_q=40, attn_lse=FAKE)   # 20 x 4 pairs
    assert status("sparse_attn_validate", ctypes.byref(big)) == UNSUPPORTED
    bad = ctypes.byref(params(block_table=FAKE, page_size=5, max_pages=1000))
    assert status("sparse_attn_append_kv", bad, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, None) == INVALID


def test_calls_reject_small_workspace():
    p = params()
    _, fwd = _ws(p)
    vp = ctypes.c_void_p
    r = status("sparse_attn_fwd", ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
               None, vp(FAKE), fwd - 1, None)
    assert r == WORKSPACE
    assert str(fwd) in _lib.lib().sparse_attn_last_error().decode()
    p = params(batch=1, max_q=4096, total_q=4096, max_k=4096, total_k=4096)
    r = status("sparse_attn_select", ctypes.byref(p), vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), None, None, 0,
               None)
    assert r == WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()


def _bx(**kw):
    b = _lib.SaBucketIndex()
    base = dict(block_tokens=512, count=64, cap_tokens=16, blocks_max=8, centroid=FAKE, member=FAKE, offset=FAKE)
    base.update(kw)
    for k, v in base.items():
        setattr(b, k, v)
    return b


@pytest.mark.parametrize("field,value,code", [
    ("block_tokens", 510, INVALID), ("block_tokens", 1024, UNSUPPORTED), ("count", 0, INVALID),
    ("count", 129, INVALID), ("cap_tokens", 8, INVALID), ("cap_tokens", 6, INVALID), ("blocks_max", 3, INVALID),
    ("centroid", None, INVALID), ("member", None, INVALID), ("centroid", FAKE + 4, INVALID),
    ("build_from", -1, INVALID)])
def test_bucket_build_rejects(field, value, code):
    p = params(block=4, max_k=4096, total_k=8192)                 # 128 groups per 512-token block
    b = _bx(**{field: value})
    vp = ctypes.c_void_p
    assert status("sparse_attn_bucket_build", ctypes.byref(p), vp(FAKE), ctypes.byref(b), None) == code
    assert _lib.lib().sparse_attn_last_error().decode()


def test_bucket_select_checks():
    p = params(block=4, max_k=4096, total_k=8192, topk=1024)
    b = ctypes.byref(_bx())
    n = ctypes.c_size_t(0)
    assert status("sparse_attn_bucket_workspace_size", ctypes.byref(p), b, 256, ctypes.byref(n)) == 0 and n.value > 0
    for nb, code in ((0, INVALID), (1025, INVALID), (257, INVALID)):     # 257 * 4 > the 1024-wide table
        assert status("sparse_attn_bucket_workspace_size", ctypes.byref(p), b, nb, ctypes.byref(n)) == code
    wide = params(block=4, max_k=4096, total_k=8192, topk=8192)
    assert status("sparse_attn_bucket_workspace_size", ctypes.byref(wide), b, 256, ctypes.byref(n)) == UNSUPPORTED
    vp = ctypes.c_void_p
    assert status("sparse_attn_bucket_select", ctypes.byref(p), vp(FAKE), b, 256, vp(FAKE), vp(FAKE), vp(FAKE), 16,
                  None) == WORKSPACE
