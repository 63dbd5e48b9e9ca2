"""Build libvjp.so for gfx950 from csrc/*.hip with hipcc (no GPU needed).

Every source is compiled to an object under _build/ in parallel, then the
objects are linked into row_wise_backward_amd/libvjp.so.  Packed fp32 VALU
instructions are disabled for device code (-packed-fp32-ops); the host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvjp.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (install ROCm or set HIPCC)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[cc, *compile_flags(), "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for cmd, fut in zip(cmds, [ex.submit(_run, c) for c in cmds]):
            fut.result()
            if verbose:
                print("compiled", cmd[-3], flush=True)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("linked", LIB, flush=True)
    return LIB


CONSUMER_SRC = os.path.join(ROOT, "tests", "c_abi_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "_build", "c_abi_consumer")


def consumer_cmd(out: str = CONSUMER, link: bool = True) -> list[str]:
    """gcc command for the plain-C99 consumer of the ABI (tests/c_abi_consumer.c):
    the header and the HIP runtime's C API only, linked against libvjp.so with
    run paths relative to the program, so the tree can move."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), CONSUMER_SRC]
    if not link:
        return cmd + ["-fsyntax-only"]
    rel = os.path.relpath(PKG, os.path.dirname(out))
    return cmd + ["-o", out, "-L", PKG, "-lvjp", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
                  f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]


def build_consumer(verbose: bool = False) -> str:
    """Compile the C consumer against the built library (after build())."""
    os.makedirs(os.path.dirname(CONSUMER), exist_ok=True)
    _run(consumer_cmd())
    if verbose:
        print("linked", CONSUMER, flush=True)
    return CONSUMER


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    build_consumer(verbose="-q" not in sys.argv)
