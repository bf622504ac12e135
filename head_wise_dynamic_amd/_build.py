"""Build libsaf3r.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled with packed-FP32 instruction selection switched
off (``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it
does not know the feature, which is harmless.
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
OUT = os.path.join(PKG, "libsaf3r.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("SAF_OFFLOAD_ARCH", "gfx950")

# (source, object, extra flags): the cosine GEMM is compiled once per phase
# mode (its instantiations dominate the build time), all units in parallel
SOURCES = [(s, os.path.splitext(s)[0], []) for s in
           ["api.cpp", "attn_mfma.hip", "attn_valu.hip", "vertical.hip", "corr_index.hip", "corr_block.hip",
            "nmse.hip", "noalloc.cpp"]]
SOURCES += [("corr_cos.hip", f"corr_cos_m{m}", [f"-DSAF_COS_MODE={m}"]) for m in range(7)]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _deps(path: str, seen=None) -> set:
    """The file and every quoted #include it reaches (csrc/ and include/)."""
    seen = set() if seen is None else seen
    if path in seen or not os.path.exists(path):
        return seen
    seen.add(path)
    for line in open(path, errors="replace"):
        m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
        if m:
            for base in (os.path.dirname(path), CSRC, os.path.join(ROOT, "include")):
                cand = os.path.normpath(os.path.join(base, m.group(1)))
                if os.path.exists(cand):
                    _deps(cand, seen)
                    break
    return seen


def _compile(unit, force: bool = True) -> str:
    src, name, extra = unit
    obj = os.path.join(BUILD, name + ".o")
    if not force and os.path.exists(obj):
        newest = max([os.path.getmtime(f) for f in _deps(os.path.join(CSRC, src))] + [os.path.getmtime(__file__)])
        if os.path.getmtime(obj) > newest:
            return obj
    cmd = ["hipcc"] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, force: bool = True) -> str:
    """Compile every source and link.  force=False reuses an object that is
    newer than its source, every header and this script."""
    os.makedirs(BUILD, exist_ok=True)
    # the slowest units first, so that they start at once
    units = sorted(SOURCES, key=lambda u: u[0] not in ("corr_cos.hip", "corr_index.hip", "attn_mfma.hip"))
    with ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(units))) as ex:
        objs = list(ex.map(lambda u: _compile(u, force), units))
    tmp = OUT + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True, force="--changed" not in sys.argv)
    sys.exit(0)
