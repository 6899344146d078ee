"""Build libsdv.so (HIP, gfx950) in-tree with hipcc.

Compile flags: -O3 for gfx950 only; packed-fp32 instructions are disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops with a leading minus).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsdv.so")
SOURCES = ["api.hip", "gemm.hip", "attention.hip", "elementwise.hip", "accept.hip", "draft.hip", "pool.hip", "streams.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, under _build/) and link."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include")]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = common + ["-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        return obj, r

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    failed = [r for _, r in results if r.returncode != 0]
    for r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed building libsdv.so")
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libsdv.so")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
