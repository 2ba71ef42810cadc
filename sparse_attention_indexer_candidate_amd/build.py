"""Build libidx.so (the C-ABI library) from csrc/ with hipcc for gfx950, in-tree."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/idx_api.hip", "csrc/idx_expand.hip", "csrc/idx_sparse.hip",
           "csrc/idx_row_groups.hip", "csrc/idx_dense.hip", "csrc/idx_gather.hip",
           "csrc/idx_measure.hip"]
LIB = os.path.join(HERE, "libidx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the ReLU-weight epilogue reads every accumulator, so
    # AGPR results would cost one extra move per element
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the leading scalar kernel arguments (up to 16 SGPRs) are preloaded at wave launch,
    # so a kernel's first loads do not wait for a load of their own addresses
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel: each is its own unit), then links
    the shared library; the objects live in a temporary folder."""
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="idx_build_") as tmpdir:
        objs, cmds = [], []
        for s in SOURCES:
            obj = os.path.join(tmpdir, os.path.basename(s) + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *FLAGS, "-c", os.path.join(HERE, s), "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for c, rc in zip(cmds, pool.map(subprocess.call, cmds)):
                if rc != 0:
                    raise subprocess.CalledProcessError(rc, c)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
