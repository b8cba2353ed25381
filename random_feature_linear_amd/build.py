"""Build libdarkprf.so (HIP, gfx950) in-tree with hipcc.

    python -m random_feature_linear_amd.build          # or build() from Python

The forward kernels are templates over (element type, head dimension, rank
blocks) and the decode kernel over (element type, head dimension).  Each
combination is compiled in a unit of its own, so that the compilations run in
parallel; those units are generated here (under _build/gen) from the tables
below.  Every .hip file under csrc/ and every generated unit is compiled and
the objects are linked into random_feature_linear_amd/libdarkprf.so.  The
library is compiled every time this runs.
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
GEN_DIR = os.path.join(OUT_DIR, "gen")
LIB = os.path.join(HERE, "libdarkprf.so")
ARCH = os.environ.get("DARKPRF_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep packed-fp32 VALU instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", f"-I{CSRC}",
]
# MFMA results in ordinary VGPRs (no accumulator-register copies around the exp)
# for the instantiations whose registers fit in 256 VGPRs; the others keep the
# accumulator registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
_UNIT = re.compile(r"fwd_(bf16|f32)_d(\d+)_r(\d+)\.hip$")

# The instantiated combinations; api.hip's dispatch tables name the same set.
DTYPES = {"bf16": "bf16", "f32": "float"}
HEAD_DIMS = (16, 32, 64, 128, 256)
RANK_BLOCKS = (1, 2, 4, 8, 16)      # geometry rank in 16-wide blocks


def feature_blocks_per_wave(d_h: int) -> int:
    """32-feature blocks per wave of the key-side kernel (the planner in
    api.hip uses the same rule)."""
    return 2 if d_h <= 64 else 1


FWD_UNIT = """\
// Forward instantiation: element type {ctype}, head dimension {dh}, rank blocks {r16}.
#include "prf_kernels.h"

namespace dk {{
dark_status fwd_{dt}_d{dh}_r{r16}(const FwdArgs& a, const Plan& p, void* ws, void* s) {{
  return launch_fwd_impl<{ctype}, {dh}, {r16}, {fbw}>(a, p, ws, s);
}}
dark_status exact_{dt}_d{dh}_r{r16}(const FwdArgs& a, void* ws, void* s) {{
  return launch_exact_impl<{ctype}, {dh}, {r16}>(a, ws, s);
}}
}}  // namespace dk
"""

DEC_UNIT = """\
// Decode instantiation: element type {ctype}, head dimension {dh}.
#include "prf_kernels.h"
#include "decode_kernels.h"

namespace dk {{
dark_status dec_{dt}_d{dh}(const dark_prf_desc& d, const void* q, const void* k, const void* v, const float* M,
                         const float* om, float* S, float* z, void* out, const uint8_t* qm, int upd, void* s) {{
  return launch_decode_impl<{ctype}, {dh}>(d, q, k, v, M, om, S, z, out, qm, upd, s);
}}
}}  // namespace dk
"""


def generate_units() -> list:
    """Write the instantiation units (only when their text changed) and return their paths."""
    os.makedirs(GEN_DIR, exist_ok=True)
    units = {}
    for dt, ctype in DTYPES.items():
        for dh in HEAD_DIMS:
            for r16 in RANK_BLOCKS:
                units[f"fwd_{dt}_d{dh}_r{r16}.hip"] = FWD_UNIT.format(
                    dt=dt, ctype=ctype, dh=dh, r16=r16, fbw=feature_blocks_per_wave(dh))
            units[f"dec_{dt}_d{dh}.hip"] = DEC_UNIT.format(dt=dt, ctype=ctype, dh=dh)
    paths = []
    for name, text in sorted(units.items()):
        path = os.path.join(GEN_DIR, name)
        old = None
        if os.path.exists(path):
            with open(path) as f:
                old = f.read()
        if old != text:
            with open(path, "w") as f:
                f.write(text)
        paths.append(path)
    return paths


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
    srcs += generate_units()
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
