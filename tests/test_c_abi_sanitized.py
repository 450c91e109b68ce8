"""The host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The host layout source (flatten, floor-rule slice, segment table, reshard plan, status strings)
includes no HIP header, so it is compiled here with g++ and the sanitizers, on a line that names
no device source, and linked with the plain-C test programs of tests/c_abi.  host_check runs the
random cases against the oracle; host_edges runs the edge cases, where every caller array is
allocated at exactly its stated capacity.  A heap overrun, a signed overflow in the offset
arithmetic or any other undefined behaviour ends the run with an error.
"""

import os
import shutil
import subprocess

import pytest

import host_check_cases

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "fsdp_sharded_optimizer_layout_amd", "csrc", "layout.cpp")
INC = os.path.join(ROOT, "include")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not available")
    out = tmp_path_factory.mktemp("asan")
    obj = str(out / "layout.o")
    cmds = [["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, f"-I{INC}", "-c", SRC,
             "-o", obj]]
    for prog in ("host_check", "host_edges"):
        cmds.append(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", *SAN, f"-I{INC}",
                     os.path.join(HERE, "c_abi", prog + ".c"), obj, "-lstdc++",
                     "-o", str(out / prog)])
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr
    return out


def test_sanitized_random_cases_match_oracle(sanitized):
    host_check_cases.check_random_cases(str(sanitized / "host_check"), env=ENV)


def test_sanitized_edge_cases(sanitized):
    r = subprocess.run([str(sanitized / "host_edges")], capture_output=True, text=True,
                       timeout=300, env=ENV)
    assert r.returncode == 0, r.stderr
    assert r.stderr == "", r.stderr
    assert r.stdout.split("\n")[:-1] == [
        "ok layout_capacity", "ok plan_capacity", "ok int64_extremes", "ok empty",
        "ok many_tensors", "ok invalid", "ok status_strings", "ok fuzz_layout", "ok fuzz_plan"]
