"""Compile the synthetic-input generator: libsynth_cpu.so (gcc) and
libsynth_dev.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_CPU = os.path.join(HERE, "libsynth_cpu.so")
LIB_DEV = os.path.join(HERE, "libsynth_dev.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_cpu(verbose=False):
    tmp = LIB_CPU + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-o", tmp, os.path.join(HERE, "synth_cpu.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_CPU)
    return LIB_CPU


def build_dev(verbose=False):
    tmp = LIB_DEV + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-o", tmp, os.path.join(HERE, "synth_dev.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_DEV)
    return LIB_DEV


def build(verbose=False):
    return build_cpu(verbose), build_dev(verbose)


if __name__ == "__main__":
    print(build(verbose=True))
