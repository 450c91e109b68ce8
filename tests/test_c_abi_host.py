"""The host entry points called from plain C (tests/c_abi/host_check.c and host_edges.c, built
with gcc against include/fsdpshard.h and libfsdpshard.so).

host_check's layout, segment table and reshard plan are checked against the oracle on random
cases; host_edges runs the edge cases (short caller arrays, int64 extremes, empty inputs, argument
errors) and checks them itself.  This shows that the header is valid C and that the C ABI works
without Python in the call path.
"""

import os
import subprocess

import pytest

import host_check_cases

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "bin")
LIB = os.path.join(os.path.dirname(HERE), "fsdp_sharded_optimizer_layout_amd", "libfsdpshard.so")
PROGRAMS = ("host_check", "host_edges")


@pytest.fixture(scope="module")
def bin_dir():
    if not os.path.exists(LIB):
        pytest.fail("libfsdpshard.so is not built")
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(HERE, "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stale = [p for p in PROGRAMS if not os.path.exists(os.path.join(BIN, p))
             or os.path.getmtime(os.path.join(BIN, p)) < os.path.getmtime(LIB)
             or os.path.getmtime(os.path.join(BIN, p)) < os.path.getmtime(
                 os.path.join(HERE, "c_abi", p + ".c"))]
    if stale:
        mod.build()
    return BIN


def test_c_program_matches_oracle(bin_dir):
    host_check_cases.check_random_cases(os.path.join(bin_dir, "host_check"))


def test_c_edge_cases(bin_dir):
    out = subprocess.run([os.path.join(bin_dir, "host_edges")], capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split("\n")[:-1] == [
        "ok layout_capacity", "ok plan_capacity", "ok int64_extremes", "ok empty",
        "ok many_tensors", "ok invalid", "ok status_strings", "ok fuzz_layout", "ok fuzz_plan"]
