"""Build libxqa.so (the HIP kernels + C-ABI) in-tree for gfx950 with hipcc."""

import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libxqa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, "xqa_kernels.hip"), os.path.join(CSRC, "xqa_select.hip"),
           os.path.join(CSRC, "xqa_noalloc.hip"), os.path.join(CSRC, "xqa_api.cpp")]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for all device code. MFMA results
# are kept in ordinary VGPRs (no AGPR copies around the softmax arithmetic).
# Up to 16 leading scalar argument dwords are preloaded into SGPRs at wave
# launch (the split kernel puts the plan's inputs there, the combine kernel
# every value it reads), so they need no load from the argument block.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE,
]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(cand) and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the shared library; returns its path. Raises on failure."""
    fd, tmp = tempfile.mkstemp(prefix=".libxqa.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [hipcc()] + COMMON_FLAGS + ["-shared", "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            # hipcc's host pass does not know the packed-fp32 feature; that note is harmless.
            lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
            if lines:
                print("\n".join(lines), file=sys.stderr)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    write_build_info()
    return LIB_PATH


def write_build_info() -> None:
    """Record what the library was built from next to it (_build_info.json, not
    versioned): the source commit when git is available, the compiler version
    and the flags, so that measurements made elsewhere can name their build."""
    import json
    import time
    info = {"built_at_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()),
            "flags": " ".join(COMMON_FLAGS[:-2]), "sources": [os.path.basename(x) for x in SOURCES]}
    try:
        r = subprocess.run(["git", "-C", REPO_DIR, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        if r.returncode == 0:
            info["git_sha"] = r.stdout.strip()
            d = subprocess.run(["git", "-C", REPO_DIR, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            info["git_dirty"] = bool(d.stdout.strip())
    except Exception:
        pass
    try:
        r = subprocess.run([hipcc(), "--version"], capture_output=True, text=True, timeout=60)
        info["hipcc_version"] = " | ".join(l.strip() for l in r.stdout.splitlines()[:2])
    except Exception:
        pass
    with open(os.path.join(PKG_DIR, "_build_info.json"), "w") as f:
        json.dump(info, f, indent=1)


def resource_usage() -> str:
    """Compiler report of VGPR/AGPR/SGPR/LDS/scratch per kernel (our own build)."""
    cmd = [hipcc()] + COMMON_FLAGS + ["--offload-device-only", "-c", "-o", os.devnull,
                                      "-Rpass-analysis=kernel-resource-usage", SOURCES[0]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(res.stderr)
    keep = [l for l in res.stderr.splitlines() if "remark" in l]
    return "\n".join(keep)


if __name__ == "__main__":
    print(build(verbose=True))
    if "--resources" in sys.argv:
        print(resource_usage())
