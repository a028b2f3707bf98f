"""Build libsa.so for gfx950 in-tree with hipcc.

    python -m paged_gqa_decode_step_amd.build [--jobs N]

Every source under csrc/ is compiled for gfx950 only, with packed-fp32 ops
switched off (the compiler may not fuse fp32 pairs into v_pk_* forms), and
linked into ``paged_gqa_decode_step_amd/libsa.so``.  Objects go to ``_build/``
at the repository root.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsa.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA operands and accumulators in VGPRs: the softmax rescales the
    # accumulators every step, and AGPR copies would cost two moves per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsa.so")


def _compile(src: str, obj: str, verbose: bool, extra=()) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + FLAGS + list(extra) + lang + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(jobs: int = 8, verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source under csrc/ and link ``out`` (default: the
    package's libsa.so); returns its path.  ``defines`` are extra ``-D``
    settings of the kernels' build-time tuning knobs (SA_PIPE, SA_KV_NT), for
    building side-by-side variants to measure."""
    tag = "".join(d.replace("=", "") for d in defines)
    bdir = os.path.join(BUILD, tag) if tag else BUILD
    os.makedirs(bdir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for f in [ex.submit(_compile, s, o, verbose, extra) for s, o in zip(srcs, objs)]:
            f.result()
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="tuning knob, e.g. -D SA_PIPE=3 (use with --out)")
    ap.add_argument("--out", default=LIB, help="output library path")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose, args.defines, args.out))


if __name__ == "__main__":
    main()
