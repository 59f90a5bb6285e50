"""Build libsparsekv.so in-tree with hipcc for gfx950 (no torch extension)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsparsekv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "attend.hip", "attend_mfma.hip", "score_step.hip", "score_obs.hip", "select.hip",
           "merge.hip", "util.hip", "gather.hip", "select_topp.hip", "topk_step.hip"]
# -amdgpu-mfma-vgpr-form: MFMA accumulators stay in VGPRs (no AGPR copies
# around the vector work on them).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# Per-source additions.  topk_step.hip: its single-lane device-scope atomics
# stay plain atomics (the atomic optimizer would fold each into a wave-wide
# one whose answer is broadcast at once, waiting for the round trip where the
# kernel means to read it much later).
EXTRA_FLAGS = {"topk_step.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, extra_sources=()) -> str:
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(OBJ, os.path.basename(path) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(path), []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(sources=None, jobs: int | None = None) -> str:
    """Compile every source and link libsparsekv.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = list(sources or SOURCES)
    jobs = jobs or min(8, len(srcs), max(1, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = "probe_read.hip"
PROBE_LIB = os.path.join(HERE, "libskvprobe.so")


def build_probe() -> str:
    """Compile and link libskvprobe.so (the bench's streaming-read probe)."""
    os.makedirs(OBJ, exist_ok=True)
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, obj], check=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(sys.argv[1:] or None))
