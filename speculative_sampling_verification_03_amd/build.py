"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_sampling_verification_03_amd.build
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = [os.path.join(CSRC, "spec_verify.hip"), os.path.join(CSRC, "ngram.hip"),
           os.path.join(CSRC, "adapt.hip")]
DEPS = SOURCES + [os.path.join(CSRC, "sv_device.h"), os.path.join(CSRC, "sv_ngram.h"),
                  os.path.join(CSRC, "sv_adapt.h"),
                  os.path.join(INCLUDE, "spec_verify.h")]

ARCH = os.environ.get("SPEC_VERIFY_ARCH", "gfx950")

# Packed fp32 arithmetic is switched off for every device pass: hand-written and
# compiler-formed packed fp32 ops are avoided on this target.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libspecverify.so)")


def build(verbose=False, extra=()):
    """Compile the library; always recompiles. Returns the path of the .so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    if verbose and r.stderr.strip():
        # the host pass warns that it does not know the packed-fp32 feature
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
