"""Build libssa.so for gfx950 in-tree with hipcc (no JIT cache, no site-packages).

    python -m long_context_block_ssa_amd._build        # or __graft_entry__.build()

Every HIP source and the C-ABI layer are compiled to objects in parallel and
linked into ``long_context_block_ssa_amd/_lib/libssa.so``.  All device code is
built with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(OUT_DIR, "libssa.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 math (v_pk_fma_f32 and friends) stays off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Per-file additions.  prefill_d128.hip: no NaN can reach its max reductions
# (rows past L are clamped to real data, masked scores are -inf), so the
# compiler need not quiet NaN inputs before each v_max.  prefill_d128_bwd.hip:
# the dk/dv kernel needs more than 256 registers, and the compiler would then
# put every MFMA accumulator in AGPRs, so the score and dP tiles that the
# vector code reads would be copied out each stage; the VGPR form keeps those
# in VGPRs and leaves the dK/dV accumulators in AGPRs.
FILE_FLAGS = {
    "prefill_d128.hip": ["-fno-honor-nans"],
    "prefill_d128_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Host-side sanitizers for the C-ABI layer only (argument validation, error
# strings): AddressSanitizer and UndefinedBehaviorSanitizer on the host pass of
# api.cpp; device code is never instrumented.  The resulting library needs the
# ASan runtime preloaded into the (uninstrumented) Python process.
SAN_LIB = os.path.join(OUT_DIR, "libssa_san.so")
SAN_OBJ_DIR = os.path.join(ROOT, "_build", "obj_san")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan"]
SAN_SOURCES = ("api.cpp",)


def asan_runtime() -> str:
    """Path of the shared ASan runtime of hipcc's clang (to LD_PRELOAD)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src: str, sanitize: bool = False) -> str:
    name = os.path.basename(src)
    san = sanitize and name in SAN_SOURCES
    obj = os.path.join(SAN_OBJ_DIR if san else OBJ_DIR, name + ".o")
    extra = SAN_FLAGS if san else []
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(name, []), *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines()
            if "warning" in ln and "packed-fp32-ops" not in ln and "recognized feature" not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Build libssa.so; with ``sanitize`` build libssa_san.so instead, whose
    C-ABI layer carries the host sanitizers (kernels are the same objects)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(SAN_OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_FLAGS if sanitize else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
