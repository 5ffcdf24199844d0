"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_sampling_verification_03_amd.build
"""
import os
import re
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


# Per-kernel resource remarks from the compiler: a kernel that uses scratch (private
# memory per lane, for spills or private arrays) runs markedly slower on MI355X (an
# 8-entry private array in the one-launch kernel cost 4% at 256 sequences and 13% at
# 1024), so the build refuses one unless SPEC_VERIFY_ALLOW_SCRATCH=1.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def scratch_kernels(remarks):
    """[(kernel, bytes per lane)] of the kernels whose remarks report scratch."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose=False, extra=()):
    """Compile the library; always recompiles. Returns the path of the .so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, RESOURCE_REMARKS, *extra, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    scratch = scratch_kernels(r.stderr)
    if scratch and os.environ.get("SPEC_VERIFY_ALLOW_SCRATCH") != "1":
        os.remove(tmp)
        raise RuntimeError("kernels using scratch: " + ", ".join(f"{k} ({b} B/lane)" for k, b in scratch))
    if verbose and r.stderr.strip():
        # the host pass warns that it does not know the packed-fp32 feature; the
        # resource remarks were checked above
        lines = [l for l in r.stderr.splitlines()
                 if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and not l.startswith(" ")]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
