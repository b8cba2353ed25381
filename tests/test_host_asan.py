"""The library's host code under AddressSanitizer, on the CPU.

Builds every unit of the library with the host pass instrumented
(-Xarch_host before each sanitizer flag; device code is built as usual) into
a temporary directory, links tests/asan/fuzz_host.cpp against it and runs the
fuzz driver: random valid and invalid descriptors through every sizing call,
compute calls that must return before any launch, the host generators and the
projection lifecycle.  A sanitizer report or a broken property fails the test.
Nothing reaches a GPU.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

from random_feature_linear_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which(b.HIPCC) is None and not os.path.exists(b.HIPCC), reason="hipcc not found")
def test_host_code_under_asan(tmp_path):
    srcs = sorted(os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC) if f.endswith(".hip"))
    srcs += b.generate_units()

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [b.HIPCC, *b.CFLAGS, *b._unit_flags(src), "-O1", *SAN, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "fuzz_host")
    driver = os.path.join(HERE, "asan", "fuzz_host.cpp")
    dobj = str(tmp_path / "fuzz_host.o")
    # the driver is plain host C++: its own compile (hipcc would build every later input as HIP)
    res = subprocess.run(["g++", "-std=c++17", "-O1", "-fsanitize=address", "-fno-omit-frame-pointer",
                          f"-I{os.path.join(ROOT, 'include')}", "-c", driver, "-o", dobj], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    cmd = [b.HIPCC, f"--offload-arch={b.ARCH}", dobj, *objs, "-Xarch_host", "-fsanitize=address", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    run = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=600)
    sys.stdout.write(run.stdout[-2000:])
    assert "AddressSanitizer" not in run.stderr, run.stderr[-6000:]
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "0 property failures" in run.stdout
