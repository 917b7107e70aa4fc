"""Build libspecverify.so for gfx950 in-tree with hipcc.

    python -m speculative_decoding_verification_verify_amd.build

Compiles every ``csrc/*.hip`` and ``csrc/*.cpp`` into one shared library next
to this file.  Each call compiles (no caching), which is what the build check
needs.
"""

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 instructions stay off: the compiler forms them from plain
    # float code, and the kernels do not need them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    srcs += sorted(glob.glob(os.path.join(HERE, "csrc", "*.cpp")))
    return srcs


def build(verbose=False, out=None, defines=()):
    """Compile the library to ``out`` (default: the in-tree library).
    ``defines``: extra NAME=VALUE macros, for measurement builds only (the
    in-tree library is always built without them)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    dst = out or LIB_PATH
    tmp = dst + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *["-D" + d for d in defines], "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % dst)
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libspecverify.so for gfx950")
    ap.add_argument("--out", default=None, help="output path (default: the in-tree library)")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="extra macro for a measurement build, e.g. SV_K_TOKEN_MAJOR=1")
    a = ap.parse_args()
    if a.define and not a.out:
        ap.error("a build with --define needs --out: the in-tree library stays the plain build")
    print(build(verbose=True, out=a.out, defines=a.define))
