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


def resource_usage():
    """Per-kernel resources of the gfx950 code as the compiler reports them
    (its kernel-resource-usage remarks): {demangled name: {"VGPRs", "SGPRs",
    "LDS", "scratch", "occupancy"}}.  Compiles the kernel files again, device
    side only, without touching the library."""
    import re
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    keys = {"VGPRs": "VGPRs", "TotalSGPRs": "SGPRs", "LDS Size [bytes/block]": "LDS",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy"}
    out = {}
    with tempfile.TemporaryDirectory(prefix="dwconv_res_") as tmp:
        for src in HIP_SOURCES:
            r = subprocess.run([hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-c",
                                os.path.join(CSRC, src), "-o", os.path.join(tmp, src + ".o"),
                                "-Rpass-analysis=kernel-resource-usage"],
                               check=True, capture_output=True, text=True)
            name = None
            for line in r.stderr.splitlines():
                m = re.search(r"remark:\s+Function Name: (\S+)", line)
                if m:
                    name = m.group(1)
                    out[name] = {}
                    continue
                m = re.search(r"remark:\s+([^:]+): (\d+) \[", line)
                if name and m and m.group(1).strip() in keys:
                    out[name][keys[m.group(1).strip()]] = int(m.group(2))
    # GNU c++filt does not know _Float16 (DF16_): demangle it as half, then rename
    names = [n.replace("DF16_", "Dh") for n in out]
    dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                         check=True).stdout.split("\n")
    return {d.replace("dwconv::(anonymous namespace)::", "").replace("half", "_Float16"): v
            for d, v in zip(dem, out.values())}


if __name__ == "__main__":
    import sys
    if "--resources" in sys.argv:
        res = resource_usage()
        print("| kernel | VGPRs | SGPRs | LDS bytes / workgroup | scratch bytes / lane | "
              "waves / SIMD |\n|---|---|---|---|---|---|")
        for k in sorted(res):
            v = res[k]
            print(f"| `{k.split('(')[0]}` | {v.get('VGPRs')} | {v.get('SGPRs')} | {v.get('LDS')} | "
                  f"{v.get('scratch')} | {v.get('occupancy')} |")
    else:
        print(build(verbose=True))
