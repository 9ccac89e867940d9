"""Build libgdn.so in-tree with hipcc for gfx950.

    python -m gated_deltanet_chunked_02_amd.build        # or build() from Python

Each translation unit is compiled separately (in parallel) into ``_build/`` and linked
into ``gated_deltanet_chunked_02_amd/libgdn.so``, next to the binding that loads it.

The gfx950 assembly of every HIP source is also generated and checked.  The build fails on
a matrix-core instruction whose accumulator input overlaps the destination of a matrix-core
instruction of another shape a few instructions earlier (e.g. 16x16x32 then 16x16x16 on
the same tile): such chains gave wrong sums on gfx950 while the compiler inserted no wait
states for them, so accumulation chains keep one instruction shape.  A destination that
partly overlaps the instruction's own accumulator input (``v[134:137] ... v[132:135]``) is
accepted: within a chain of one shape it was checked on gfx950, back-to-back, with wait
states, and with two chains interleaved so that one overwrites the other's input.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["api.cpp", "stages.hip", "fused.hip", "segment.hip", "recurrent.hip", "conv1d.hip",
           "noalloc.hip", "backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: libgdn needs ROCm's hipcc to build")
    return path


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function",
            # keep packed-fp32 VALU forms out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


_MFMA = re.compile(r"^\s*(v_mfma\S*)\s+([av])\[(\d+):(\d+)\],\s*[^,]+,\s*[^,]+,\s*"
                   r"([av])\[(\d+):(\d+)\]")


def mfma_partial_overlaps(asm: str):
    """(line number, text) of every matrix-core instruction whose destination register range
    partly overlaps its accumulator-input range (same register file, not identical)."""
    bad = []
    for n, line in enumerate(asm.splitlines(), 1):
        m = _MFMA.match(line)
        if not m:
            continue
        _, df, d0, d1, cf_, c0, c1 = m.groups()
        d0, d1, c0, c1 = int(d0), int(d1), int(c0), int(c1)
        if df == cf_ and (d0, d1) != (c0, c1) and d0 <= c1 and c0 <= d1:
            bad.append((n, line.strip()))
    return bad


_MFMA_DST = re.compile(r"^\s*(v_mfma\S*)\s+([av])\[(\d+):(\d+)\],")


_FIRST_REG = re.compile(r"^\s*(\S+)\s+([av])(?:(\d+)\b|\[(\d+):(\d+)\])")
_READS_FIRST = ("ds_write", "ds_store", "buffer_store", "global_store", "flat_store",
                "scratch_store", "s_")


def mfma_mixed_chains(asm: str, window: int = 16):
    """(line number, text) of every matrix-core instruction with an accumulator-input register
    last written by a matrix-core instruction of another opcode at most `window`
    instructions earlier (labels, directives and comments not counted).  Any other
    instruction whose first operand is a vector register (its destination; stores excepted)
    counts as that register's last writer."""
    bad = []
    # (register file, number) -> (instruction index, opcode) of its last writer; opcode None
    # for a writer that is not a matrix-core instruction
    last = {}
    k = 0
    for n, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        k += 1
        m = _MFMA.match(line)
        if m:
            op, _, _, _, cf_, c0, c1 = m.groups()
            for r in range(int(c0), int(c1) + 1):
                prev = last.get((cf_, r))
                if prev is not None and prev[1] is not None and k - prev[0] <= window \
                        and prev[1] != op:
                    bad.append((n, t))
                    break
        d = _MFMA_DST.match(line)
        if d:
            for r in range(int(d.group(3)), int(d.group(4)) + 1):
                last[(d.group(2), r)] = (k, d.group(1))
            continue
        w = _FIRST_REG.match(line)
        if w and not w.group(1).startswith(_READS_FIRST):
            r0 = int(w.group(3) if w.group(3) is not None else w.group(4))
            r1 = int(w.group(3) if w.group(3) is not None else w.group(5))
            for r in range(r0, r1 + 1):
                last[(w.group(2), r)] = (k, None)
    return bad


# Per-source extra flags (none at present: LLVM's max-ILP scheduling strategy, measured on
# the fused kernel, made it about 9 % slower on gfx950).
EXTRA = {}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    if src.endswith(".hip"):
        asm = os.path.join(BUILD, os.path.splitext(src)[0] + "." + ARCH + ".s")
        cmd = [hipcc()] + flags() + EXTRA.get(src, []) + ["--cuda-device-only", "-S",
                                                          os.path.join(CSRC, src), "-o", asm]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, res.stderr))
        with open(asm) as f:
            text = f.read()
        bad = mfma_mixed_chains(text)
        if bad:
            raise RuntimeError("%s: %d matrix-core instruction(s) with an accumulator input from "
                               "a matrix-core instruction of another shape just before, e.g. "
                               "%s:%d: %s" % (src, len(bad), asm, bad[0][0], bad[0][1]))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libgdn.so; always rebuilds.  Returns the path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
