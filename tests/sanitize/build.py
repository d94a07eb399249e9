"""Build the AddressSanitizer + UndefinedBehaviorSanitizer host build of
libdit's sources with the ABI check driver (host code sanitized, device code
as usual), into _build/sanitize/abi_checks.

    python tests/sanitize/build.py        # (re)build what is out of date

Objects are rebuilt only when a source or header is newer than them."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "diffusion_transformer_dit_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "sanitize")
EXE = os.path.join(OUT, "abi_checks")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-I", INCLUDE, "-I", CSRC]


def _newest(paths):
    return max(os.path.getmtime(p) for p in paths)


def _compile(src, headers):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    if os.path.exists(obj) and os.path.getmtime(obj) >= _newest([src, *headers]):
        return obj
    r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    headers = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(HERE, "abi_checks.cpp")]
    jobs = min(len(srcs), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, headers), srcs))
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < _newest(objs):
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], "-o", EXE, *objs], capture_output=True,
                           text=True)
        if r.returncode:
            raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    return EXE


if __name__ == "__main__":
    print(build())
    sys.exit(0)
