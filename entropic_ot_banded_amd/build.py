"""Build libsinkattn.so (HIP for gfx950) in place, next to this file.

    python -m entropic_ot_banded_amd.build [--debug]

Compiles csrc/*.hip and csrc/api.cpp with hipcc (in parallel) into one shared
library.
Packed fp32 VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libsinkattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    out = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    out.append(os.path.join(CSRC, "api.cpp"))
    return out


def build(debug: bool = False, verbose: bool = False) -> str:
    """Compile every source into libsinkattn.so; returns the library path.
    Sources compile in parallel (one object each), then link."""
    import concurrent.futures
    import tempfile

    flags = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-O1" if debug else "-O3", "-I", INCLUDE,
             "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]
    tmpdir = tempfile.mkdtemp(prefix="sinkattn_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc()] + flags + ["-c", "-x", "hip", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        srcs = sources()
        jobs = max(1, min(len(srcs), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, srcs))
        for (obj, res), src in zip(results, srcs):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed compiling {os.path.basename(src)}")
        tmp = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libsinkattn.so")
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, verbose=True))
