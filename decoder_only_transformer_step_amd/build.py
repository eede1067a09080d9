"""Compile libdecoder.so (the HIP kernels and the C ABI) for gfx950.

Each HIP source compiles to its own object in parallel (a temporary folder
beside the library), then one link makes the shared library."""
import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdecoder.so")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(verbose=False):
    tmp = tempfile.mkdtemp(prefix="_build_", dir=HERE)
    try:
        srcs = sources()
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        cmds = [["hipcc"] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
                for s, o in zip(srcs, objs)]
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        msgs = []
        for (rc, m), s in zip(results, srcs):
            msgs += m
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(s)}:\n" + "\n".join(m))
        rc, m = _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"])
        msgs += m
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(m))
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
