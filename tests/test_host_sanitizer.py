"""Host-sanitizer build: the library's host code and the C oracle under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The MetaInfer-cpp (Qwen3 C++ Reference Runtime) README keeps a Debug host
sanitizer build among its performance-hardening gates.  Here the packer's
pointer loops, the C ABI's argument validation and the oracle are rebuilt
with the sanitizers (device code unchanged), and the CPU tests that drive
them (tests/test_host_abi.py, the oracle pins and the argmax pins) run again
in a child process that preloads clang's ASan runtime and loads the
sanitized libraries (QG_LIBRARY, ORACLE_LIBRARY).  A planted overflow (a
packer told its output buffer is larger than it is) must be reported, which
shows the sanitizer is live in that process.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not ASAN_RT, reason="clang's shared ASan runtime is not installed")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    sys.path.insert(0, ROOT)
    import oracle
    from weight_only_block_amd import build
    out = str(tmp_path_factory.mktemp("asan"))
    lib = build.build(verbose=False, out_dir=out, sanitize=True)
    olib = oracle.build_sanitized(os.path.join(out, "liboracle.so"))
    logs = os.path.join(out, "report")
    env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], QG_LIBRARY=lib, ORACLE_LIBRARY=olib,
               PYTHONPATH=ROOT, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:log_path=" + logs,
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:log_path=" + logs)
    return env, logs


def _reports(logs):
    text = ""
    for f in glob.glob(logs + "*"):
        with open(f) as fh:
            text += fh.read()
        os.remove(f)
    return text


def test_host_tests_pass_under_sanitizers(sanitized):
    env, logs = sanitized
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_host_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_argmax.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = _reports(logs)
    assert r.returncode == 0 and not reports, (reports + r.stdout + r.stderr)[-6000:]


def test_planted_packer_overflow_is_reported(sanitized):
    code = (
        "import numpy as np\n"
        "from weight_only_block_amd import qgemv as Q\n"
        "q = np.zeros((64, 128), np.int8); s = np.zeros((64, 2), np.uint16)\n"
        "size = Q.qpack_q8g64_size(64, 128)\n"
        "out = np.empty(size - 512, np.uint8)\n"
        "Q.lib().qpack_q8g64(Q._np_ptr(q), Q._np_ptr(s), 64, 128, Q._np_ptr(out), size)\n")
    env, logs = sanitized
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    reports = _reports(logs)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in reports
    assert "pack_q8" in reports
