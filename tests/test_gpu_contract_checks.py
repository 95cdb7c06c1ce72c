"""The library built with contract checks (libsparse_attn_checked.so; needs an MI355X).

Its kernels validate what they gather through the caller's device tables (sequence
geometry, selection tables, block tables, token positions) and report violations as
bits read by sparse_attn_check_flags, taking clamped in-range indices instead.  The
scenarios run in one child process that loads the checked library
(tests/contract_check_run.py): valid calls on every workload's small shape set no bit
and meet the oracle's bars; each planted violation sets its own bit.
"""
import os
import subprocess
import sys

import pytest

import top_block_sparse_mean_amd as sa
from top_block_sparse_mean_amd import build

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def results():
    assert os.path.exists(build.CHECKED_OUT), "build the checked library first (__graft_entry__.build())"
    env = dict(os.environ, SPARSE_ATTN_LIB=build.CHECKED_OUT)
    r = subprocess.run([sys.executable, os.path.join(HERE, "contract_check_run.py")], env=env,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    lines = [ln.split() for ln in r.stdout.splitlines() if ln.strip()]
    assert lines[-1] == ["done"]
    return {name: int(v) for name, v in lines[:-1]}


def test_valid_calls_set_no_flag(results):
    valid = {k: v for k, v in results.items() if k.startswith("valid_")}
    assert len(valid) >= 7
    assert all(v == 0 for v in valid.values()), valid


@pytest.mark.parametrize("case,bit", [("bad_entry", sa.SA_CHECK_TABLE), ("bad_count", sa.SA_CHECK_TABLE),
                                      ("bad_page", sa.SA_CHECK_PAGE)])
def test_planted_violation_sets_its_bit(results, case, bit):
    assert results[case] & bit, results[case]
    assert not results[case] & sa.SA_CHECK_SEQ, results[case]
