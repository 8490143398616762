"""Build libattn.so (the C-ABI attention library) for gfx950 with hipcc.

Usage: ``python -m scaled_dot_product_09_amd.build`` (or ``build()`` from
Python). Always recompiles. The library is written next to this file, in the
source tree, so it travels with the tree.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd_mfma.hip", "attn_fwd_f32.hip", "attn_combine.hip", "attn_bwd.hip", "attn_fp8_scaling.hip", "attn_noalloc.hip"]

# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU ops
# (v_pk_fma_f32 and friends); every HIP source is built with it.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Device code only: no NaN canonicalisation around min/max (the kernels
    # never create NaN from finite inputs; NaN inputs are outside the
    # supported domain). Host code keeps full IEEE semantics for validation.
    "-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


# Per-source flags. The backward kernels keep every matrix-product result
# that the vector ALU reads in ordinary VGPRs (MFMA "VGPR form"); the default
# puts them in accumulation registers, and the copies back cost more than
# the products (measured: +29 % on the head-dim-64 backward). The forward
# kernel's score accumulators are read by the vector ALU too.
SOURCE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "attn_fwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=True, extra_flags=()):
    """Compile every source to an object (with its own flags), link libattn.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmpdir:
        objs = [os.path.join(tmpdir, src + ".o") for src in SOURCES]
        cmds = [[hipcc(), *compile_flags, *SOURCE_FLAGS.get(src, []), *extra_flags, "-I",
                 os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
                for src, obj in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
