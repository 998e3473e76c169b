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
HOST_SOURCES = ["host.cpp", "cpu_step.cpp"]      # host C++ only (built by the host compiler)
DEVICE_SOURCES = ["shard_step.hip", "combine.hip", "copy_ref.hip", "hbm_alloc.hip"]   # HIP: host launchers + gfx950 kernels
SOURCES = HOST_SOURCES + DEVICE_SOURCES
ARCH = "gfx950"

COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fno-math-errno", "-Wall"]
# Packed fp32 VALU forms are disabled: the compiler emits plain fp32 ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def host_cxx() -> str:
    return os.environ.get("HOST_CXX", "/opt/rocm/bin/amdclang++")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
    if verbose and res.stderr.strip():
        sys.stderr.write("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l) + "\n")


def build(verbose: bool = False, out_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the library; returns its path.  Raises CalledProcessError."""
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory() as tmpdir:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            _run([host_cxx(), "-x", "c++", *COMMON_FLAGS, "-pthread", *inc, *extra_flags, "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        for src in DEVICE_SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            _run([hipcc(), f"--offload-arch={ARCH}", *COMMON_FLAGS, "-Wno-unused-command-line-argument", *inc,
                  *DEVICE_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
        os.close(fd)
        try:
            _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp], verbose)
            os.replace(tmp, out_path)
        finally:
            if os.path.exists(tmp):
                os.unlink(tmp)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
