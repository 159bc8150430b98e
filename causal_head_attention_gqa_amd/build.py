"""Build the gfx950 HIP library libattn_gfx950.so in-tree with hipcc.

Usage: python -m causal_head_attention_gqa_amd.build   (or build() from Python)
Every source is compiled each time (the build is the "does it compile" check); objects go to
_build/ at the repository root, the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn_gfx950.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code (the compiler would otherwise form
# v_pk_* from ordinary float code); the host pass ignores the feature with a warning.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)$")


def _regs(tok: str):
    m = _REG.match(tok.strip())
    if not m:
        return None
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def mfma_overlaps(asm: str) -> list[str]:
    """Matrix-core instructions whose destination registers overlap their A or B operand.

    The compiler may allocate an MFMA's destination over a source that dies at the instruction;
    on gfx950 such code has produced run-to-run different results, so the build rejects it (the
    kernels keep their sources live through the mfma wrappers in common.hpp instead).
    """
    bad = []
    for line in asm.splitlines():
        t = line.strip()
        if not t.startswith("v_mfma"):
            continue
        ops = t.split(None, 1)[1].split(",")
        d, a, b = (_regs(o) for o in ops[:3])
        for s in (a, b):
            if d and s and d[0] == s[0] and not (d[2] < s[1] or s[2] < d[1]):
                bad.append(t)
                break
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    asm = os.path.join(BUILD, os.path.basename(src)[:-4] + ".s")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    r = subprocess.run([HIPCC, *FLAGS, "--cuda-device-only", "-S", src, "-o", asm], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(asm) as f:
        bad = mfma_overlaps(f.read())
    if bad:
        raise RuntimeError(f"{src}: MFMA destination overlaps a source operand:\n" + "\n".join(bad[:5]))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
