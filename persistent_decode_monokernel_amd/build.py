"""Build libkie.so from the HIP sources of csrc/ for gfx950 with hipcc.

Each translation unit is compiled in its own hipcc process (in parallel), then
the objects are linked into one shared library.

Usage: python -m persistent_decode_monokernel_amd.build [--verbose]
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkie.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep packed fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(SRC, f) for f in os.listdir(SRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, msgs


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", SRC]
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, *extra, *inc, "-c", src, "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, msgs) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd))
        if rc != 0:
            raise RuntimeError(f"hipcc failed for {obj} ({rc}):\n{msgs}")
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *[o for o, _ in jobs]])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
