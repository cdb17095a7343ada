"""Build libswa.so (HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m sliding_window_attention_amd.build``.  Always recompiles.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libswa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["swa_api.hip", "fwd_bf16.hip", "fwd_f32.hip", "split_kv.hip", "rope.hip"]

# The bf16 kernels never create NaNs (masked scores are -inf, never NaN), so
# they are built without IEEE NaN quieting: fmax then needs no canonicalising
# moves in front of every MFMA result.  Infinities stay honoured.  (Such code
# cannot inline the device-library accessors behind threadIdx / blockIdx, so
# these sources read the ids through the hardware builtins instead.)
RELAXED_NAN = {"fwd_bf16.hip", "split_kv.hip"}

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep hipcc from emitting packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-variable",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        extra = ["-fno-honor-nans", "-mno-amdgpu-ieee"] if src in RELAXED_NAN else []
        cmds.append([HIPCC] + FLAGS + extra + inc + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # one hipcc per source, side by side
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
