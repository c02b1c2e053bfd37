"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_mixture_experts_softmax_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["route_topk.hip", "route_grouped.hip", "align_sort.hip", "expert_map.hip", "quant_act.hip", "experts_gemm.hip", "gemm_lds.hip", "moe_abi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: the compiler may not form v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int = 8, out: str = LIB, defines=()) -> str:
    """Compile every source and link `out`.  `defines` are extra -D macros (tuning
    knobs that have defaults in the sources)."""
    build_dir = BUILD_DIR if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
