"""Build the HIP library dense_gemm_07_amd/lib/libdg.so for gfx950.

Every translation unit is compiled by hipcc (in parallel) into _build/, then
linked into one shared library exporting the C-ABI of include/dg.h.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdg.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dg_host.cpp", "simt.hip", "split_reduce.hip", "attention.hip", "mfma_f32.hip"] + [
    f"mfma_{t}_{m}.hip" for t in ("bf16", "f16") for m in ("kc_rc", "kc_kc", "rc_rc", "rc_kc", "gn", "unaligned")]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-unit flags. The attention kernel's accumulators stay in ordinary VGPRs
# (gfx950 MFMA reads and writes them directly): in accumulation registers every
# softmax step would copy its scores and rescale its output through
# v_accvgpr_read / v_accvgpr_write.
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 0, only=None) -> str:
    """Compile every unit (or, with `only`, just those units, reusing the other
    objects from an earlier build) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    todo = SOURCES if not only else [s for s in SOURCES if s in only]
    if only and len(todo) != len(set(only)):
        raise ValueError(f"unknown sources in {only}")
    jobs = jobs or min(len(todo), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"objects missing (run a full build): {missing}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    only = next((a.split("=", 1)[1].split(",") for a in sys.argv if a.startswith("--only=")), None)
    print(build(verbose="-v" in sys.argv, only=only))
