"""Builds libmoe.so (the HIP library, gfx950) and the device input generator
libsynth.so with hipcc, in-tree."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth_device.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynth.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: every f32/f64 operation is rounded as written (FMAs only where
# spelled out); the packed-FP32 feature is off (its forms are not trusted here).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-command-line-argument"]
SOURCES = ["moe_api.hip", "moe_route.hip", "moe_experts.hip", "moe_decode1.hip", "moe_prefill.hip",
           "moe_shared_pf.hip", "moe_cache.hip", "moe_score_table.hip"]
# the prefill kernels consume MFMA results in VALU code: keep them in VGPRs (no accvgpr copies);
# the single-token kernels' leading scalar arguments are preloaded into SGPRs at wave launch
EXTRA = {"moe_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "moe_decode1.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    synth_obj = os.path.join(BUILD, "synth_device.o")
    cmds.append([HIPCC, *FLAGS, "-c", SYNTH_SRC, "-o", synth_obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", synth_obj, "-o", tmp], verbose)
    os.replace(tmp, SYNTH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
