"""Build libheal.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

The library is written in-tree next to this file, so it travels with the
source tree.  hipcc cross-compiles for gfx950 without a GPU present.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libheal.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


# per-source additions: the attention kernels keep their MFMA accumulators in
# ordinary VGPRs (no AGPR round trip before the softmax and rescale math, and
# fewer registers in all)
PER_SOURCE = {
    "attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, obj: str, extra, verbose: bool):
    cmd = [HIPCC, *FLAGS, *extra, *PER_SOURCE.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC, "-c",
           src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, extra=()) -> str:
    """Compile each source to an object (in parallel), then link the shared
    library.  Every object carries its own gfx950 code object."""
    import concurrent.futures
    import tempfile
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="heal_build_") as td:
        srcs = sources()
        objs = [os.path.join(td, os.path.basename(s) + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            results = list(ex.map(lambda so: _compile(so[0], so[1], extra, verbose), zip(srcs, objs)))
        for src, r in zip(srcs, results):
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed compiling {os.path.basename(src)}")
            if verbose and r.stderr.strip():
                sys.stderr.write(r.stderr)
        cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libheal.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
