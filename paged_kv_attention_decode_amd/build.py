"""Build libpkv.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# source -> extra flags.  The prefill kernel's MFMA accumulators take the
# vector-register form: left in the accumulation registers, the rare rescale of
# the running output made the compiler copy accumulators out and back around
# its branch on every tile.
SOURCES = {
    "pkv_kernels.hip": [],
    "pkv_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "pkv_pages.hip": [],
    "pkv_probe.hip": [],
    "pkv_api.cpp": [],
}


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source of the library (always) and link it."""
    tmpdir = tempfile.mkdtemp(prefix="pkv_build_")
    try:
        inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
        procs, objs = [], []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [HIPCC, *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, p in procs:
            out, err = p.communicate()
            if p.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out + err)
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd))
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
