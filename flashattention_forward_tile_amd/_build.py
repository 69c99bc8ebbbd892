"""Build the HIP library libfa2.so (gfx950 only) in the package directory."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa2_fwd.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa2.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code; the softmax and
# epilogue arithmetic is plain scalar-per-lane fp32.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path


def compile_cmd(out, extra=()):
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-shared", "-I", INCLUDE, *DEVICE_FLAGS, *extra, "-o", out, SRC]


def build(verbose: bool = False, extra=()) -> str:
    """Compile csrc/fa2_fwd.hip into libfa2.so and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = compile_cmd(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
