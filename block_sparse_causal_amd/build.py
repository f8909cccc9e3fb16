"""Compile libstem.so in-tree for gfx950 with hipcc.

    python -m block_sparse_causal_amd.build

Every HIP source under csrc/ and the host planning code are linked into one
shared library next to this file.  Packed-FP32 instruction selection is
turned off for device code (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstem.so")
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + \
        sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the host code
# (planning, argument checks); every flag goes to the host compilation only,
# the GPU code is built as usual.  The resulting library expects the ASan
# runtime to be preloaded (see sanitizer_runtime).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc (preloaded into the
    process that loads a sanitized library)."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True).stdout.strip()
    return out


def build(verbose: bool = False, extra_flags=None, out: str = None, sanitize: bool = False) -> str:
    """Compile every source into libstem.so (always recompiles); ``out``
    builds elsewhere, ``sanitize`` adds the host sanitizers."""
    lib = out or LIB
    tmp = lib + ".tmp"
    flags = list(extra_flags or []) + (SANITIZE_HOST if sanitize else [])
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp] + flags + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is expected and carries no information.
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in proc.stdout.splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
