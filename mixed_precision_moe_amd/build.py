"""Build the HIP library libmoe.so for gfx950 (in-tree).

    python -m mixed_precision_moe_amd.build

Every .hip source under csrc/ is compiled with hipcc for gfx950 and linked
into mixed_precision_moe_amd/libmoe.so.  Packed fp32 vector instructions are
disabled for all device code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 8) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        objs, procs = [], []
        for src in srcs:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *FLAGS, "-I", os.path.join(HERE, "..", "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0 or (verbose and out.strip()):
                print(out, file=sys.stderr)
            if p.returncode != 0:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
