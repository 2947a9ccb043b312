"""Build libpagedkv.so for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_03_amd.build        # or build() from Python

Every call compiles from source (no cache check), each .hip file in its own
hipcc process, then links the shared library next to this file.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
SOURCES = ["api.hip", "pa_decode.hip", "pa_decode_flat.hip", "pa_decode_grouped.hip", "pa_prefill.hip", "cache_ops.hip", "probe.hip", "vkv.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is needed to build libpagedkv")
    return path


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, save_temps=False):
    """Compile every source for gfx950 and link PKG_DIR/libpagedkv.so.
    Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "--save-temps")
        objs.append(obj)
        cmds.append(cmd)
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        logs = list(ex.map(_run, cmds))
    lib = os.path.join(PKG_DIR, LIB_NAME)
    tmp = lib + ".tmp"
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]))
    os.replace(tmp, lib)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
