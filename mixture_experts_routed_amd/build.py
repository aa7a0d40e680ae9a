"""Build the HIP library libmoe_routed.so for gfx950 (MI355X), in-tree.

hipcc compiles every kernel source and the C-ABI translation unit to an
object (in parallel), then links one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_routed.so")
SOURCES = ["route.hip", "plan.hip", "gather_combine.hip", "ffn.hip", "stage.hip", "abi.cpp",
           "noalloc.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    # the host pass does not know the gfx950-only feature name; drop that notice
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if msg.strip() and verbose:
        print(msg)


def build(verbose: bool = False, host_flags=(), lib: str = LIB, build_dir: str = BUILD) -> str:
    """Build the library at `lib`. host_flags are added to the host compilation only
    (each passed behind -Xarch_host), e.g. the tests' AddressSanitizer build of the
    host code; the device code is the same either way."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    xhost = [a for f in host_flags for a in ("-Xarch_host", f)]
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(build_dir, s.replace(".", "_") + ".o")
        objs.append(o)
        cmds.append([cc, *FLAGS, *xhost, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *xhost, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
