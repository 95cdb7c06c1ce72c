"""Host code under address and undefined-behaviour sanitizers (CPU only).

The library is rebuilt with host-side checks (the GPU code as usual) and the host
ABI tests run against it with the sanitizer runtime preloaded: every validation,
sizing and error path of the C ABI executes under the checks.  The oracle is
rebuilt the same way with gcc and every pin runs against it.  A report from
either sanitizer fails the test.
"""
import os
import subprocess
import sys

from top_block_sparse_mean_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

ASAN = "detect_leaks=0:exitcode=99"
UBSAN = "halt_on_error=1:print_stacktrace=1:exitcode=98"

PINS = r"""
import sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import pins
failed = []
for p in pins.ALL:
    try:
        p()
    except Exception as e:
        failed.append(f"{p.__name__}: {e!r}"[:300])
print("FAILED PINS:", failed)
sys.exit(1 if failed else 0)
"""


def _clean(r):
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]


def test_host_abi_under_sanitizers(tmp_path):
    so = build.build(sanitize=True, out=str(tmp_path / "libsparse_attn_san.so"), build_dir=str(tmp_path / "obj"))
    env = dict(os.environ, SPARSE_ATTN_LIB=so, LD_PRELOAD=build.sanitizer_runtime(), ASAN_OPTIONS=ASAN,
               UBSAN_OPTIONS=UBSAN)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_host.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    _clean(r)
    assert " passed" in r.stdout and "failed" not in r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           str(so), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, ORACLE_LIB=str(so), LD_PRELOAD=asan, ASAN_OPTIONS=ASAN, UBSAN_OPTIONS=UBSAN,
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", PINS, ROOT, HERE], env=env, capture_output=True, text=True,
                       timeout=900)
    _clean(r)
