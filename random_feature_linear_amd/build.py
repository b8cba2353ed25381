"""Build libdarkprf.so (HIP, gfx950) in-tree with hipcc.

    python -m random_feature_linear_amd.build          # or build() from Python

Every .hip unit under csrc/ is compiled in parallel and linked into
random_feature_linear_amd/libdarkprf.so.  The library is compiled every time
this runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdarkprf.so")
ARCH = os.environ.get("DARKPRF_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep packed-fp32 VALU instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# MFMA results in ordinary VGPRs (no accumulator-register copies around the exp)
# for the instantiations whose registers fit in 256 VGPRs; the others keep the
# accumulator registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
_UNIT = re.compile(r"fwd_(bf16|f32)_d(\d+)_r(\d+)\.hip$")


def _unit_flags(src: str) -> list:
    m = _UNIT.search(os.path.basename(src))
    if m and int(m.group(2)) <= 128 and int(m.group(3)) <= 4:
        return VGPR_FORM
    return []


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *_unit_flags(src), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr[-6000:]}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = jobs or max(1, min(16, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} units", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
