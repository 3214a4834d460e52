"""Build of the DeltaKV HIP library (libdeltakv.so, gfx950) in this package
directory.  Run as ``python -m residual_kv_cache_amd.build_lib``.

Each source compiles to its own object in ``_build/`` (in parallel: the
kernel files take minutes each), then the objects are linked into the
shared library.  No device code is shared across files, so no relocatable
device code is needed."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdeltakv.so")
SOURCES = ["api.hip", "compress.hip", "decode.hip", "decode_mfma.hip", "append.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    return res.returncode, msgs


def _stale(src: str, obj: str) -> bool:
    """An object is out of date when it is missing or older than its source
    or any header of the library."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    return any(os.path.getmtime(p) > t for p in deps)


def build(verbose: bool = False, jobs: int = 0, incremental: bool = False) -> str:
    """Compile every source into libdeltakv.so.  Always rebuilds every object
    unless ``incremental`` (then only objects older than their inputs)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)
            if not incremental or _stale(os.path.join(CSRC, s), o)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(max(1, len(cmds)), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    errors = []
    for cmd, (rc, msgs) in zip(cmds, results):
        if rc != 0:
            errors.append(f"{os.path.basename(cmd[-3])}:\n" + "\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs))
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
