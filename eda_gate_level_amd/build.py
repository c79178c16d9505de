"""Build the gfx950 shared library libpa.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.hip", "pa_load.hip", "pa_pass.hip"]
HOST_SOURCES = ["pa_text.cpp"]  # plain C++ (the activity-text packer), built with the host compiler
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere (hipcc's host pass warns that it
    # does not know this feature; that warning is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libpa.so (always rebuilds)."""
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(CSRC, src.replace(".cpp", ".o"))
        cmd = ["g++", "-O3", "-std=c++17", "-fPIC", "-pthread", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
               "-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    try:
        failed = None
        for cmd, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out)
                failed = failed or cmd
            elif verbose and out:
                sys.stderr.write(out)
        if failed:
            raise RuntimeError(f"hipcc failed: {' '.join(failed)}")
        tmp = LIB + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs]
        subprocess.run(link, check=True)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
