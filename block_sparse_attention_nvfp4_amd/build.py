"""Build libmsa.so (the HIP kernels and the C ABI of include/msa.h) in-tree for gfx950, and its
checked variant libmsa_checked.so (the same sources with MSA_CHECKED: the kernels also count
failed checks of their device-memory inputs and index arithmetic, include/msa_debug.h).

    python block_sparse_attention_nvfp4_amd/build.py      # or build() of __graft_entry__

(run as a file: importing the package loads the library it builds)

Each .hip file under csrc/ is compiled by hipcc to an object and the objects are linked into
block_sparse_attention_nvfp4_amd/libmsa.so (objects in _build/) and libmsa_checked.so (objects
in _build_checked/). Packed-fp32 instructions are disabled for all device code; there is no
fast-math, so fp32 division and square root stay IEEE-rounded.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmsa.so")
CHECKED_BUILD_DIR = os.path.join(HERE, "_build_checked")
CHECKED_LIB = os.path.join(HERE, "libmsa_checked.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the first kernel arguments arrive in scalar registers with the wavefront (no memory load
    # at kernel start where the firmware supports it; the code falls back to loading them)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MSA library needs the ROCm toolchain")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *defines, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def _link(objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Build both libraries; returns the path of libmsa.so."""
    variants = ((BUILD_DIR, LIB, ()), (CHECKED_BUILD_DIR, CHECKED_LIB, ("-DMSA_CHECKED",)))
    for build_dir, _, _ in variants:
        os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = [(s, d, defs) for d, _, defs in variants for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs))
    for i, (_, lib, _) in enumerate(variants):
        _link(objs[i * len(srcs):(i + 1) * len(srcs)], lib, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
