"""Build the HIP library ``libfa.so`` in-tree for gfx950.

    python -m exact_attention_05_amd.build      # or: python exact_attention_05_amd/build.py
    python -m exact_attention_05_amd.build --incremental

Compiles every ``csrc/*.hip`` with hipcc (in parallel) and links them into
``exact_attention_05_amd/lib/libfa.so``.  Packed-fp32 VALU instructions are
disabled for all device code.  With ``--incremental`` an object newer than
its source and every header is kept.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
OUT = os.path.join(OUT_DIR, "libfa.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # Device code only: NaN inputs are not supported (they propagate
        # unchecked), so the compiler need not quiet NaNs before every max;
        # infinities are still honoured (the masks use -inf).  Host code keeps
        # full IEEE semantics for argument validation.
        "-Xarch_device", "-fno-honor-nans",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


# Per-source code-generation options (none at present).
FILE_FLAGS: dict[str, list[str]] = {}


def _headers() -> list[str]:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    return hs + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]


def _up_to_date(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return False
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(f) < t for f in [src, *_headers(), os.path.abspath(__file__)])


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    if incremental and _up_to_date(src, obj):
        return obj
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *compile_flags(), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is expected, anything else is shown.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True, incremental: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, incremental), srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:])
