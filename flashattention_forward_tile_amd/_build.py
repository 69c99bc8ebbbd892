"""Build the HIP library libfa2.so (gfx950 only) in the package directory."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa2_fwd.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa2.so")
# The race-check build of the same source (tests only): every load waited
# where it is issued, so its results must equal libfa2.so's bit for bit.
LIB_SYNC = os.path.join(PKG, "libfa2_sync.so")
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


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile csrc/fa2_fwd.hip into `out` (libfa2.so) and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = compile_cmd(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sync(verbose: bool = False) -> str:
    """Compile the race-check build into libfa2_sync.so."""
    return build(verbose, extra=("-DFA2_SYNC_CHECK=1",), out=LIB_SYNC)


if __name__ == "__main__":
    print(build(verbose=True))
