"""Build libdwconv.so in-tree: host C++ with g++, kernels with hipcc for gfx950.

``build()`` always recompiles (a stale library is worse than a slow build).
"""
import concurrent.futures
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdwconv.so")
HOST_SOURCES = ["dwconv_api.cpp", "dwconv_plan.cpp"]
HIP_SOURCES = ["dwconv_direct.hip", "dwconv_tiled_nhwc.hip", "dwconv_tiled_nchw.hip",
               "dwconv_wgrad.hip", "dwconv_launch.hip", "dwconv_stream.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra_hipcc=()) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    with tempfile.TemporaryDirectory(prefix="dwconv_build_") as tmp:
        objs = []
        for src in HOST_SOURCES:
            o = os.path.join(tmp, src + ".o")
            _run(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", o], verbose)
            objs.append(o)
        # the kernel files compile independently: one hipcc each, in parallel
        hip_objs = [os.path.join(tmp, src + ".o") for src in HIP_SOURCES]
        jobs = max(1, min(len(HIP_SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, [hipcc, *HIPCC_FLAGS, *extra_hipcc, "-c",
                                         os.path.join(CSRC, src), "-o", o], verbose)
                      for src, o in zip(HIP_SOURCES, hip_objs)]:
                f.result()
        objs += hip_objs
        out_tmp = LIB + ".tmp"
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp, *objs],
             verbose)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
