"""Build libmamba3.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m state_space_sequence_prefill_amd.build

Compiles every source of the library with hipcc into objects under _build/
(in parallel) and links them into state_space_sequence_prefill_amd/libmamba3.so,
and the bandwidth probes of the measurement harness (csrc/m3_probe.hip) into
libm3probe.so beside it.  Always recompiles.  No GPU is needed: hipcc
cross-compiles for gfx950.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmamba3.so")
PROBE_LIB = os.path.join(PKG, "libm3probe.so")
PROBE_SOURCES = ["m3_probe.hip"]
SOURCES = ["m3_api.cpp", "m3_state.hip", "m3_decode.hip", "m3_decode_mimo.hip", "m3_prefill.hip", "m3_prefill_pc.hip",
           "m3_prefill_pc_gated.hip", "m3_prefill_pc_down.hip", "m3_prefill_pc_bcnorm.hip",
           "m3_prefill_pc_bcnorm_gated.hip", "m3_prefill_pc_bcnorm_down.hip", "m3_backward.hip",
           "m3_backward_bf16.hip", "m3_backward_f32.hip", "m3_noalloc.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmamba3.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Packed fp32 instructions stay off: plain fp32 code only.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU target feature; drop that notice.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
