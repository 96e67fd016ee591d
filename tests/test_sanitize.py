"""The library's host codec and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/blob_fuzz.cpp is built with -fsanitize=address,undefined (host
code only: host_codec.cpp, nwc_oracle.c and the driver; no device code) and
run on a bounded number of random matrices, parameter sets and mutated blobs:
the library's and the oracle's encoders must write identical bytes that
decode back exactly, and neither parser may crash on a mutated blob (any
sanitizer report aborts the run with a non-zero status).  The encode/decode
and validation logic it covers is otherwise tested through the Python
bindings of the unsanitized builds.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    d = tmp_path_factory.mktemp("san")
    orc = str(d / "nwc_oracle.o")
    subprocess.run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "nwc_oracle.c"), "-o", orc],
                   check=True)
    exe = str(d / "blob_fuzz")
    subprocess.run(["g++", "-std=c++17", *SAN, "-pthread", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "decode_gemv_byte_amd", "csrc"),
                    os.path.join(ROOT, "tests", "sanitize", "blob_fuzz.cpp"),
                    os.path.join(ROOT, "decode_gemv_byte_amd", "csrc", "host_codec.cpp"), orc, "-o", exe, "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_codec_and_oracle_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, "150", str(seed)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "no failure" in r.stdout
