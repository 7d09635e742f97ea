"""Builds libssu.so (the gfx950 kernels and the C-ABI entry points) in-tree
with hipcc."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssu.so")
SOURCES = [os.path.join(CSRC, "ssu_kernels.hip"), os.path.join(CSRC, "ssu_replay.hip"),
           os.path.join(CSRC, "ssu_copy.hip"),
           os.path.join(CSRC, "ssu_ssd.hip"), os.path.join(CSRC, "ssu_noalloc.hip"),
           os.path.join(CSRC, "ssu_api.cpp")]
# Streaming-ceiling kernels for the benchmark (a separate library, not part
# of libssu's interface).
CEILING_SRC = os.path.join(CSRC, "ssu_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libssu_ceiling.so")
HEADERS = [os.path.join(CSRC, "ssu_internal.h"), os.path.join(CSRC, "ssu_device.h"),
           os.path.join(os.path.dirname(HERE), "include", "ssu.h")]

# Packed-fp32 instructions are switched off for all device code; hipcc -O3
# still vectorises loads, stores and conversions.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fvisibility=hidden"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out=LIB, extra=(), ceiling=True):
    """Compile the library into `out` (always recompiles), and the ceiling
    library next to the package; returns `out`.

    Each source is compiled to its own object in parallel (no relocatable
    device code: every translation unit carries its own kernels), then the
    objects are linked."""
    tag = "%s.%d" % (os.path.basename(out), os.getpid())
    srcs = SOURCES + ([CEILING_SRC] if ceiling else [])
    objs = [os.path.join(os.path.dirname(out), "_%s_%s.o" % (os.path.basename(src), tag))
            for src in srcs]

    def compile_one(i):
        subprocess.run([hipcc(), *HIPCC_FLAGS, *extra, "-c", "-o", objs[i], srcs[i]], check=True)

    def link(lib, parts):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *parts],
                       check=True)
        os.replace(tmp, lib)

    try:
        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "4"))))
        with ThreadPoolExecutor(jobs) as pool:
            list(pool.map(compile_one, range(len(srcs))))
        link(out, objs[:len(SOURCES)])
        if ceiling:
            link(CEILING_LIB, objs[len(SOURCES):])
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


def stale(lib=LIB):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build())
