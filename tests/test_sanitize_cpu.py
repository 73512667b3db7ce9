"""The oracle and the C-ABI host layer under the host compiler's address and
undefined-behaviour sanitizers (CPU only).

* The oracle (oracle/tsel_oracle.c) is built with gcc -fsanitize=address,
  undefined, and its pin tests run against that build.
* The host layer of libtsel.so (tsel_api.cpp: argument checks, on-chip
  layout planning, kernel choice, workspace carving) is built with g++ and
  the same sanitizers against stand-in launchers that run no kernel
  (tests/sanitize/launch_stubs.cpp), and the ABI tests run against it.

Both run in a child process with the sanitizer runtime preloaded; any
report aborts it (-fno-sanitize-recover)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "logits_processing_token_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-shared", "-fPIC"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None
                                or not os.path.isdir("/opt/rocm/include"),
                                reason="needs gcc, g++ and the HIP headers")

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import pytest
import oracle
oracle._lib = oracle.bind({oracle_so!r})
from logits_processing_token_amd import tsel
tsel.LIB_PATH = {host_so!r}
sys.exit(pytest.main({args!r}))
"""


def test_oracle_and_host_layer_under_sanitizers(tmp_path):
    oracle_so = str(tmp_path / "liboracle_san.so")
    host_so = str(tmp_path / "libtsel_host_san.so")
    subprocess.check_call(["gcc", *SAN, "-o", oracle_so,
                           os.path.join(ROOT, "oracle", "tsel_oracle.c"), "-lm"])
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                           "-I" + CSRC, "-o", host_so, os.path.join(CSRC, "tsel_api.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")])
    files = ["test_oracle_rules.py", "test_oracle_bruteforce.py", "test_oracle_logprob.py",
             "test_oracle_verify_select.py", "test_oracle_beam.py", "test_abi.py"]
    args = [os.path.join(ROOT, "tests", f) for f in files] + [
        "-q", "-x", "-m", "not gpu", "-k", "not planted", "-p", "no:cacheprovider"]
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = CHILD.format(root=ROOT, oracle_so=oracle_so, host_so=host_so, args=args)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
