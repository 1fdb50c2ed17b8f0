"""Build libkvs.so in-tree with hipcc for gfx950.

    python block_sparse_kv_amd/build.py              # libkvs.so
    python block_sparse_kv_amd/build.py --timeline   # libkvs_timeline.so: the same library with
                                                     # per-workgroup timeline records (-DKVS_TIMELINE),
                                                     # loaded when KVS_LIBRARY=timeline

Every .hip / .cpp file under csrc/ is compiled to an object of its own (in parallel, under _build/)
and the objects are linked into one shared library next to this file.  Packed-fp32 instructions are
disabled for the device code (-packed-fp32-ops); the host pass warns that it does not know that
feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvs.so")
LIB_TIMELINE = os.path.join(HERE, "libkvs_timeline.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if NOISE not in ln)
    return r.returncode, err


def build(verbose: bool = True, timeline: bool = False) -> str:
    """Compile every source into libkvs.so, or with timeline into libkvs_timeline.so (always
    recompiles); returns the library path."""
    obj_dir = OBJ + ("_timeline" if timeline else "")
    lib = LIB_TIMELINE if timeline else LIB
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    defs = ["-DKVS_TIMELINE"] if timeline else []
    jobs = []
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        jobs.append((src, obj, [HIPCC, *FLAGS, *defs, *inc, "-c", src, "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    if verbose:
        print(f"hipcc {' '.join(FLAGS)} -c <each of {len(jobs)} sources> ({workers} jobs)", flush=True)
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[2]), jobs))
    for (src, _, _), (rc, err) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
        if err.strip() and verbose:
            print(err, flush=True)
    tmp = lib + ".tmp"
    rc, err = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[1] for j in jobs]])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
