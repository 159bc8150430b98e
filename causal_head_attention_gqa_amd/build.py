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


_BFE = re.compile(r"^s_bfe_i64\s+(s\[\d+:\d+\]),")
_LDS_SADDR = re.compile(r"^global_load_lds_dword\w*\s+v\d+,\s*(s\[\d+:\d+\])")


def sign_extended_lds_bases(asm: str, window: int = 8) -> list[str]:
    """Direct-to-LDS loads whose 64-bit SGPR base was built by a signed 32-to-64-bit extension.

    A base pointer rebuilt from two 32-bit halves must zero-extend its low word; a sign
    extension (s_bfe_i64 ..., 0x200000) turns every address whose bit 31 is set into an address
    in the top 4 GiB, i.e. a memory fault. The scan looks a few instructions ahead of each
    s_bfe_i64 for a global_load_lds that takes the same register pair as its base.
    """
    lines = [ln.strip() for ln in asm.splitlines()]
    bad = []
    for i, t in enumerate(lines):
        m = _BFE.match(t)
        if not m:
            continue
        for u in lines[i + 1:i + 1 + window]:
            n = _LDS_SADDR.match(u)
            if n and n.group(1) == m.group(1):
                bad.append(t + " -> " + u)
                break
    return bad


_SREG = re.compile(r"s\[(\d+):(\d+)\]|s(\d+)$")


def _sgprs(tok: str):
    m = _SREG.match(tok.strip())
    if not m:
        return None
    if m.group(1):
        return int(m.group(1)), int(m.group(2))
    return int(m.group(3)), int(m.group(3))


def valu_sgpr_lds_hazards(asm: str, wait_states: int = 5) -> list[str]:
    """Direct-to-LDS loads whose SGPR base pair was written by a VALU instruction fewer than 5
    wait states earlier.

    A VMEM instruction that reads an SGPR written by a VALU instruction (v_readfirstlane_b32,
    v_readlane_b32, a v_cmp into an SGPR pair) needs 5 wait states in between; the compiler
    inserts them for the loads it emits itself but not in front of inline assembly, where a
    stale base gives wrong addresses. Walking back from each load, each instruction counts one
    wait state and s_nop N counts N + 1; a scalar instruction that writes part of the pair
    settles that part. A label inside the window ends the walk with the pair still unsettled,
    which is reported too (another predecessor may have written it).
    """
    lines = [ln.strip() for ln in asm.splitlines()]
    no_dest = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
               "s_sleep", "s_endpgm", "s_dcache", "s_sendmsg")
    bad = []
    for i, t in enumerate(lines):
        n = _LDS_SADDR.match(t)
        if not n:
            continue
        lo, hi = _sgprs(n.group(1))
        open_regs = set(range(lo, hi + 1))
        ws = 0
        for u in reversed(lines[:i]):
            if not u or u.startswith(";"):  # comments, including "; %bb.N:" of fall-through blocks
                continue
            if u.endswith(":"):  # a branch target (compiler labels start with "." too)
                bad.append("label " + u + " within the wait window of " + t)
                break
            if u.startswith("."):  # directives
                continue
            parts = u.split(None, 1)
            d = _sgprs(parts[1].split(",")[0]) if len(parts) > 1 and not u.startswith(no_dest) else None
            if d:
                hit = open_regs & set(range(d[0], d[1] + 1))
                if hit and u.startswith("v_"):
                    bad.append(u + " -> " + t)
                    break
                open_regs -= hit
                if not open_regs:
                    break
            m = re.match(r"s_nop\s+(\d+)", u)
            ws += int(m.group(1)) + 1 if m else 1
            if ws >= wait_states:
                break
    return bad


_LDS_DMA = re.compile(r"^global_load_lds_dword")


def m0_lds_dma_hazards(asm: str) -> list[str]:
    """Direct-to-LDS loads that come too soon after an instruction that writes M0.

    The load takes its LDS address from M0. A scalar instruction that writes M0 needs 1 wait
    state before such a load, and a vector instruction that writes it (v_readfirstlane_b32 m0,
    ...) needs 5. The compiler inserts these only in front of the loads it emits itself, not in
    front of inline assembly, which is how the kernels issue these loads. Walking back from each
    load, each instruction counts one wait state and s_nop N counts N + 1. The walk ends when a
    scalar write of M0 is found at a safe distance, or after 5 wait states. A write found closer
    than its hazard needs is reported, and so is a label reached before the walk ends (another
    predecessor may have written M0).
    """
    lines = [ln.strip() for ln in asm.splitlines()]
    bad = []
    for i, t in enumerate(lines):
        if not _LDS_DMA.match(t):
            continue
        ws = 0
        for u in reversed(lines[:i]):
            if not u or u.startswith(";"):  # comments, including "; %bb.N:" of fall-through blocks
                continue
            if u.endswith(":"):  # a branch target (compiler labels start with "." too)
                bad.append("label " + u + " within the M0 wait window of " + t)
                break
            if u.startswith("."):  # directives
                continue
            parts = u.split(None, 1)
            dest = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
            if dest == "m0":
                if u.startswith("v_"):
                    bad.append(u + " -> " + t)  # any vector write within 5 wait states
                elif ws < 1:
                    bad.append(u + " -> " + t)
                break
            m = re.match(r"s_nop\s+(\d+)", u)
            ws += int(m.group(1)) + 1 if m else 1
            if ws >= 5:
                break
    return bad


def scan(text: str) -> list[tuple[str, list[str]]]:
    """Every check of the generated assembly, as (what is wrong, offending lines) pairs."""
    return [
        ("MFMA destination overlaps a source operand", mfma_overlaps(text)),
        ("sign-extended base address of a direct-to-LDS load", sign_extended_lds_bases(text)),
        ("direct-to-LDS load reads an SGPR a VALU wrote < 5 wait states earlier", valu_sgpr_lds_hazards(text)),
        ("direct-to-LDS load too soon after an M0 write", m0_lds_dma_hazards(text)),
    ]


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
        text = f.read()
    for what, bad in scan(text):
        if bad:
            raise RuntimeError(f"{src}: {what}:\n" + "\n".join(bad[:5]))
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
