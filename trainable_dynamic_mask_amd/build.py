"""Build the gfx950 HIP library of the DMA forward in-tree (libdma_hip.so).

Every .hip/.cpp file under csrc/ is compiled with hipcc for gfx950 and linked
into one shared library next to this file, and once more with DMA_SAFE_SYNC
into libdma_hip_safe.so (the synchronisation cross-check, used by the tests).
Packed fp32 VALU instructions are disabled for all device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdma_hip.so")
LIB_SAFE = os.path.join(HERE, "libdma_hip_safe.so")
OBJ = os.path.join(HERE, "_build")
ARCH = os.environ.get("DMA_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src, obj_dir, extra):
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose=False, jobs=8):
    """Build libdma_hip.so and its cross-check twin libdma_hip_safe.so (the same
    sources with DMA_SAFE_SYNC: every barrier of the hand-synchronised attention
    waits for all loads in flight, for bit-for-bit comparison in the tests)."""
    variants = ((LIB, OBJ, []), (LIB_SAFE, OBJ + "_safe", ["-DDMA_SAFE_SYNC"]))
    tasks = []
    for _, obj_dir, extra in variants:
        os.makedirs(obj_dir, exist_ok=True)
        tasks += [(src, obj_dir, extra) for src in sources()]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda t: _compile(*t), tasks))
    if verbose:
        for obj, msgs in results:
            if msgs.strip():
                print(msgs)
    for lib, obj_dir, _ in variants:
        objs = [o for o, _ in results if os.path.dirname(o) == obj_dir]
        tmp = lib + ".tmp"
        subprocess.run(["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
