"""The CPU side of the codec under AddressSanitizer and UndefinedBehaviorSanitizer (host compiler
only; nothing runs on a GPU).

tests/sanitize/fuzz_main.cpp drives the oracle (compress / decompress round trips in every
container, ragged widths, 64 and 128 lanes, refinement, escapes), the library's host tile encoder
against the oracle's, and a mutation fuzz of the blob parsers -- the library's ep_blob_parse,
which takes untrusted bytes, and the oracle's -- over every blob: byte flips, header fields set
to extreme values, truncations, rewritten table records and offsets.  The library's host code
(ep_host.cpp) and the oracle are compiled with the sanitizers; the device-code objects are the
ones the library build produced (linked only to resolve symbols; no kernel is launched)."""

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "entropy_coded_weight_ep_amd", "csrc")
BUILD = os.path.join(ROOT, "entropy_coded_weight_ep_amd", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-O1", "-g"]


@pytest.mark.timeout(600)
def test_host_code_and_oracle_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    objs = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
    if not objs:
        pytest.skip("the library is not built (run __graft_entry__.build())")
    d = str(tmp_path)
    run = lambda cmd: subprocess.run(cmd, check=True, capture_output=True, text=True)
    run(["gcc", "-c", *SAN, "-std=c11", "-ffp-contract=off", "-fno-fast-math",
         "-o", f"{d}/oracle.o", os.path.join(ROOT, "oracle", "ep_oracle.c")])
    run(["g++", "-c", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", f"{d}/host.o",
         os.path.join(CSRC, "ep_host.cpp")])
    run(["g++", "-c", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "oracle"), "-o", f"{d}/main.o",
         os.path.join(ROOT, "tests", "sanitize", "fuzz_main.cpp")])
    run(["g++", *SAN[:2], "-o", f"{d}/fuzz", f"{d}/main.o", f"{d}/host.o", f"{d}/oracle.o",
         *objs, "-L/opt/rocm/lib", "-lamdhip64", "-lpthread", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([f"{d}/fuzz"], capture_output=True, text=True, env=env, timeout=500)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "0 failures" in res.stdout
