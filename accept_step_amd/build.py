"""Build the HIP library ``libspecverify.so`` in-tree for gfx950.

    python -m accept_step_amd.build        (or accept_step_amd.build.build())

Compiles ``csrc/specverify.hip`` with hipcc.  Packed-FP32 instructions are
disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspecverify.so")
SRC = os.path.join(HERE, "csrc", "specverify.hip")


def hipcc_command(out=LIB, arch="gfx950", host_sanitizers=False):
    """The hipcc command line of the library.  ``host_sanitizers``: a checking build of
    the host code only (AddressSanitizer and UndefinedBehaviorSanitizer, each flag
    passed to the host compilation alone; device code unoptimised, to build quickly),
    for CPU tests of the argument and workspace logic.  Never for GPU runs."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    opt = ["-O1", "-Xarch_device", "-O0"] if host_sanitizers else ["-O3"]
    san = []
    if host_sanitizers:
        for f in ("-g", "-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer",
                  "-fno-sanitize-recover=undefined"):
            san += ["-Xarch_host", f]
        san.append("-shared-libasan")
    return [hipcc, f"--offload-arch={arch}"] + opt + ["-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"] + san + [
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            "-o", out, SRC]


def build(verbose=False):
    """Compile the library (always recompiles); returns its path."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libspecverify.so")
    if verbose and r.stderr:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
