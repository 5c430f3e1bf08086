"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into liblocks.so.

Run ``python -m kv_cache_page_rank_amd.build`` (the repository's build entry
point calls it too).
Packed-fp32 instructions are disabled on purpose: the compiler otherwise
forms v_pk_*_f32 from ordinary float code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblocks.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


# Extra flags of the summary-scan translation units: MFMA results in ordinary
# VGPRs (the kernel fits two waves per SIMD either way, and the VALU reads the
# results without accumulator-register moves), and no IEEE NaN handling (the
# scan's max/exp chains then need no canonicalising moves; the scan never
# reads NaN: rows of absent pages are zeroed by their bit patterns).
SCAN_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"]
EXTRA_FLAGS = {"scan_f32.hip": SCAN_FLAGS, "scan_bf16.hip": SCAN_FLAGS, "scan_q8q4.hip": SCAN_FLAGS}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the gfx feature flag: drop that one warning
    noise = [ln for ln in res.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln
             and "warning generated" not in ln and "warnings generated" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = OUT + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
