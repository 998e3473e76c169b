"""Compile libzero_shard.so in-tree with hipcc for gfx950 (MI355X).

    python -m zero_sharded_mixed_partition_amd.build

builds every source under csrc/ into one shared library next to this file.
The library is C-ABI only: the Python side loads it with ctypes.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libzero_shard.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["host.cpp", "shard_step.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled: the compiler emits plain fp32 ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, out_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the library; returns its path.  Raises CalledProcessError."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
           *DEVICE_FLAGS, *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
        if verbose and res.stderr.strip():
            sys.stderr.write(res.stderr)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
