"""Compile the generator: libsynth.so (host, gcc + OpenMP) and
libsynth_dev.so (device, hipcc for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host():
    src = os.path.join(HERE, "synth.c")
    out = os.path.join(HERE, "libsynth.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", out, src, "-lm"])
    return out


def build_device():
    src = os.path.join(HERE, "synth_dev.hip")
    out = os.path.join(HERE, "libsynth_dev.so")
    res = subprocess.run(["hipcc"] + HIP_FLAGS + ["-o", out, src], capture_output=True, text=True)
    if res.returncode != 0:
        msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    return out


def build():
    return build_host(), build_device()


if __name__ == "__main__":
    print(build())
