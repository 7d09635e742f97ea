"""Builds libssu.so (the gfx950 kernels and the C-ABI entry points) in-tree
with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssu.so")
SOURCES = [os.path.join(CSRC, "ssu_kernels.hip"), os.path.join(CSRC, "ssu_copy.hip"),
           os.path.join(CSRC, "ssu_ssd.hip"),
           os.path.join(CSRC, "ssu_api.cpp")]
HEADERS = [os.path.join(CSRC, "ssu_internal.h"),
           os.path.join(os.path.dirname(HERE), "include", "ssu.h")]

# Packed-fp32 instructions are switched off for all device code; hipcc -O3
# still vectorises loads, stores and conversions.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fvisibility=hidden"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out=LIB, extra=()):
    """Compile the library into `out` (always recompiles); returns `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def stale(lib=LIB):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build())
