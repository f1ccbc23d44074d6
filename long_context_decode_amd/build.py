"""Build liblcd.so (HIP kernels + C ABI) for gfx950 in-tree.

    python long_context_decode_amd/build.py [--jobs N] [--verbose]

Each source under csrc/ is compiled to an object in csrc/_build/ with hipcc, then
linked into long_context_decode_amd/liblcd.so with only the lcd_* symbols
exported.  Packed-fp32 instructions are disabled for every device compile.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "liblcd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["lcd_host.cpp", "scratch.hip", "kv.hip", "decode.hip", "snapkv.hip", "h2o_prompt.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool, defines=(), out_dir=OUT_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *[f"-D{d}" for d in defines], "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(jobs: int | None = None, verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile and link; ``defines`` are extra -D macros (kernel variants), ``out``
    the library path (default: the in-tree liblcd.so the package loads)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out_dir = OUT_DIR if not defines else os.path.join(OUT_DIR, "_".join(d.replace("=", "") for d in defines))
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, out_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           f"-Wl,--version-script={os.path.join(CSRC, 'exports.map')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    shutil.move(tmp, out)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra macro for an experimental build, e.g. -D NAME=1")
    ap.add_argument("--out", default=LIB, help="library path (default: the in-tree liblcd.so)")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, tuple(a.defines), a.out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
