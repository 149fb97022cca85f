"""Build libmha.so in-tree with hipcc for gfx950.

    python -m transformer_head_scaled_amd.build        # or build() from Python

Every call recompiles every source (it is the "does it build" check as well
as the build).  The result is transformer_head_scaled_amd/_lib/libmha.so.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmha.so")
SOURCES = ["mha_api.cpp", "sdpa_route.cpp", "sdpa_fwd.hip", "sdpa_window.hip", "sdpa_wide.hip", "sdpa_decode.hip",
           "gemm_proj.hip", "add_norm.hip", "mha_short.hip"]
# Per-source flags.  The flash attention kernel is scheduled with LLVM's
# "max-memory-clause" strategy: the same instructions and results, measured
# (interleaved runs) 1-2 % faster causal at d 64 and 128 and 2 % unmasked at
# d 128, unchanged unmasked at d 64; the default, "max-ilp" and
# "iterative-ilp" strategies measured no better.
SOURCE_FLAGS = {
    "sdpa_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "sdpa_window.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmha)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # packed fp32 VALU ops are avoided on this hardware; the device
            # compiler otherwise forms them from scalar float code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in ordinary VGPRs: the softmax rescales
            # them with VALU ops, which AGPR-resident accumulators would turn
            # into copy traffic
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src, obj, extra):
    cmd = [hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + common_flags() + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the device feature; drop that noise
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops" not in ln and "--hip-link" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose=False, extra=None):
    """Compile every source and link _lib/libmha.so.  Returns its path."""
    extra = list(extra or [])
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        futs = [ex.submit(_compile, s, o, SOURCE_FLAGS.get(s, []) + extra) for s, o in zip(SOURCES, objs)]
        for s, f in zip(SOURCES, futs):
            msg = f.result()
            if verbose and msg.strip():
                print(f"[{s}]\n{msg}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
