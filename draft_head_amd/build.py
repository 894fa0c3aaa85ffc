"""Compile the HIP sources into draft_head_amd/libdomino.so for gfx950.

Each source file is compiled to an object of its own, in parallel, then the
objects are linked into one shared library.
"""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdomino.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: hipcc would otherwise fuse fp32 pairs by itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no fused multiply-adds unless written: every kernel variant then rounds
    # the same expression the same way, and the schedules agree to the bit
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Builds the library (extra_flags / out: a differently configured copy, e.g. for tracing)."""
    obj_dir = OBJ_DIR if out == LIB else OBJ_DIR + "_" + os.path.basename(out).replace(".", "_")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + ".o")
        jobs.append((src, [HIPCC, *FLAGS, *extra_flags, *inc, "-c", src, "-o", obj], obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (src, cmd, _), (rc, err) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
        if err.strip() and verbose:
            print(err, flush=True)
    tmp = out + ".tmp"
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, _, o in jobs], "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
