"""The C ABI used from plain C99: tests/c/abi_consumer.c includes only
include/ll_moe.h, links libllmoe.so and the oracle's C library, and runs with
no Python or PyTorch in the process.

The host checks (layout sizes and offsets against the oracle, status strings,
argument errors) need no GPU; the gpu checks run a small dispatch and combine
on both parities and compare the whole layout byte for byte and the combine
output bit for bit with the oracle, then the expert side and the two-phase
combine the same way."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_ll_moe_amd")
ORACLE = os.path.join(ROOT, "oracle")
SRC = os.path.join(ROOT, "tests", "c", "abi_consumer.c")


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    for lib in (os.path.join(PKG, "libllmoe.so"), os.path.join(ORACLE, "libllmoe_oracle.so")):
        if not os.path.exists(lib):
            pytest.fail(f"{lib} is not built: run __graft_entry__.build() first")
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path_factory.mktemp("c") / "abi_consumer")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include", SRC,
           "-o", exe, "-L", PKG, "-l:libllmoe.so", "-L", ORACLE, "-l:libllmoe_oracle.so",
           "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}:{ORACLE}:/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"C consumer did not build:\n{r.stderr}"
    return exe


def _run(exe, mode):
    r = subprocess.run([exe, mode], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_c_consumer_host(consumer):
    _run(consumer, "host")


@pytest.mark.gpu
def test_c_consumer_gpu(consumer):
    print("C consumer: dispatch, combine, expert side and two-phase combine, N=37 h=384 E=9 K=3, "
          "bf16 and fp8, both parities", flush=True)
    _run(consumer, "gpu")
