"""Builds libhga.so (gfx950 only) in this package directory with hipcc.

    python hierarchical_sparse_attention_summaries_amd/build.py
    python hierarchical_sparse_attention_summaries_amd/build.py --phase-stamps

(--phase-stamps builds libhga_phases.so instead: the same library with the
one-launch decode step writing a clock stamp at the end of each of its phases;
the binding loads it when HGA_LIB names it, for `bench.py --phases`.)

(Run it as a script: importing the package loads the library it builds.)

Every source under csrc/ is compiled to an object file in parallel, then
linked into one shared library with a plain C ABI (include/hga.h).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhga.so")
BUILD = os.path.join(ROOT, "_build")
OUT_PHASES = os.path.join(PKG, "libhga_phases.so")
BUILD_PHASES = os.path.join(ROOT, "_build_phases")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # Packed fp32 instructions stay off: ordinary scalar fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def header_abi_version() -> int:
    """HGA_ABI_VERSION as include/hga.h defines it: the version a freshly built
    library must report."""
    with open(os.path.join(ROOT, "include", "hga.h")) as f:
        m = re.search(r"^#define HGA_ABI_VERSION (\d+)\s*$", f.read(), flags=re.M)
    if not m:
        raise RuntimeError("include/hga.h defines no HGA_ABI_VERSION")
    return int(m.group(1))


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True, phase_stamps: bool = False) -> str:
    build_dir = BUILD_PHASES if phase_stamps else BUILD
    out = OUT_PHASES if phase_stamps else OUT
    extra = ["-DHGA_PHASE_STAMPS"] if phase_stamps else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(phase_stamps="--phase-stamps" in sys.argv[1:])
