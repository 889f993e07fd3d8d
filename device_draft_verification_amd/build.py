"""Compile the HIP library libspecverify.so for gfx950 with hipcc.

Every kernel and the C ABI live in csrc/; the result is placed next to this
file, where the Python binding loads it from. Flags:
  -ffp-contract=off    no implicit multiply-add fusion: x = fl32(z * fl32(1/T))
                       must round exactly once, as the definition states;
  -fhip-fp32-correctly-rounded-divide-sqrt   1/T is correctly rounded;
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 ALU ops.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, jobs: int = 4, out: str | None = None,
          extra_flags=()) -> str:
    """Compile every source in csrc/ and link the library at `out` (default:
    next to this file). extra_flags are added to each compile (the sanitizer
    test passes host-only sanitizer flags)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    lib_path = out or LIB_PATH
    objdir = os.path.join(os.path.dirname(lib_path), "_build" if out is None else "_build_extra")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra_flags, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


def _wait(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out.decode(errors="replace")))
        elif out:
            text = out.decode(errors="replace")
            # hipcc's host pass does not know the packed-fp32 feature; that note is expected
            lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
            if any(ln.strip() for ln in lines):
                print("\n".join(lines))
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")


if __name__ == "__main__":
    print(build(verbose=True))
