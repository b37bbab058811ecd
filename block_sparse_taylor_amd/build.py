"""Build libpisa.so (gfx950) in-tree with hipcc.

    python -m block_sparse_taylor_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled for gfx950 only. Packed-fp32 VALU
instructions are disabled for device code (the host pass warns that it does
not know the feature; that is harmless).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpisa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source extra flags. The fused forward kernel is a long MFMA + VALU + memory
# instruction stream per wave (one wave per SIMD); the iterative ILP scheduler
# interleaves it better than the default occupancy-driven one (about 3%).
SOURCE_FLAGS = {
    "attn_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into libpisa.so; returns its path. Always rebuilds."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra_flags,
               "-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and noise:
            print("\n".join(noise))
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel whose host stub is undefined was silently dropped by the host
    # compilation pass; refuse such a library instead of failing at load time.
    nm = shutil.which("nm")
    if nm:
        undef = subprocess.run([nm, "-u", tmp], capture_output=True, text=True).stdout
        stubs = [ln.split()[-1] for ln in undef.splitlines() if "__device_stub__" in ln]
        if stubs:
            os.remove(tmp)
            raise RuntimeError(f"host pass dropped kernels (undefined stubs): {stubs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
