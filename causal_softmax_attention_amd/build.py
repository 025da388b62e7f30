"""Build libattn.so (the gfx950 HIP kernels and their C ABI) in-tree.

Usage: python causal_softmax_attention_amd/build.py [--verbose]
(run as a script: importing the package first would look for the library)

Each csrc/*.hip file is compiled by hipcc for gfx950 into an object under
_build/, then linked into causal_softmax_attention_amd/libattn.so.  Packed
fp32 instructions are disabled for the device code (-packed-fp32-ops); the
host pass reports that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]

# Per-file extra flags.  decode.hip, fwd.hip and bwd2*.hip: keep MFMA
# accumulators in VGPRs; the default AGPR form makes the compiler copy
# accumulators between register files around branches inside the loops (and
# spills in the widest backward kernels).  The large-head forward kernel
# (fwd_wide.hip, fwd_large_qk*.hip) keeps its O accumulators in AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {
    "decode.hip": VGPR_FORM,
    "prefill_paged.hip": VGPR_FORM,
    "fwd.hip": VGPR_FORM,
    "bwd2.hip": VGPR_FORM,
    "bwd2_qk128.hip": VGPR_FORM,
    "bwd2_qk256.hip": VGPR_FORM,
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer build of the C ABI (argument validation,
# workspace layout, launch set-up).  Only the host pass is instrumented: each
# sanitizer flag sits behind -Xarch_host, so the gfx950 code objects are the
# ordinary ones.  Load it with the ASan runtime preloaded (asan_runtime()).
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libattn.so")
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the ASan build links against."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    import glob
    for pat in ("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    raise RuntimeError("clang ASan runtime not found")


def build_asan(verbose: bool = False) -> str:
    """The library with the host code of api.hip built under ASan (the
    kernels' objects are shared with the regular build, built first)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = []
    for src in sources():
        base = os.path.basename(src)
        if base != "api.hip":
            obj = os.path.join(BUILD, base + ".o")
            if not os.path.exists(obj):
                _compile(src, verbose)
            objs.append(obj)
            continue
        obj = os.path.join(ASAN_DIR, base + ".o")
        cmd = [hipcc(), *COMMON_FLAGS, *ASAN_HOST_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed for {src}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_HOST_FLAGS, *objs, "-o", ASAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{r.stdout}{r.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv))
