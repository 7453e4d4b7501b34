"""Build the gfx950 HIP library libmfl_gemm.so in-tree with hipcc.

    python mma_fragment_layouts_tn_amd/_build.py

Sources are compiled in parallel to objects under ``_build/`` and linked
into ``mma_fragment_layouts_tn_amd/libmfl_gemm.so``.  The generated code of
the GEMM kernels is checked for accumulator accesses that the compiler did
not separate from the matrix instructions by the required wait states.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmfl_gemm.so")
OBJDIR = os.path.join(os.path.dirname(PKG), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gemm_inst_256.hip", "gemm_inst_256w4.hip", "gemm_inst_128.hip",
           "gemm_inst_128w1.hip", "gemm_inst_splitk.hip", "gemm_inst_256w4x16.hip",
           "gemm_inst_256x16.hip", "gemm_inst_128x16.hip", "gemm_inst_splitk16.hip", "chain_inst.hip", "gemm_dispatch.hip", "probe_kernels.hip", "microbench.hip", "probe_dump.hip", "capi.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# The generated code of every GEMM instance source is checked
# (check_mfma_fences); kernels that issue v_mfma_f32_16x16x32_f16 with the
# accumulator tied by hand (inline assembly), whose hazards the compiler
# cannot see, more strictly.
CHECKED_SOURCES = {"gemm_inst_256w4x16.hip", "gemm_inst_256x16.hip", "gemm_inst_128x16.hip",
                   "gemm_inst_splitk16.hip",
                   "gemm_inst_256.hip", "gemm_inst_256w4.hip", "gemm_inst_128.hip",
                   "gemm_inst_128w1.hip", "gemm_inst_splitk.hip", "probe_dump.hip"}
TIED_MFMA = "v_mfma_f32_16x16x32_f16"


ACC_ACCESS = re.compile(r"^v_accvgpr_(read|write|mov)")
LABEL = re.compile(r"^\.LBB\S+:$")
TERMINATOR = re.compile(r"^(s_branch|s_cbranch_\w+|s_endpgm|s_setpc_b64)\b")


def _kernels(asm_text: str) -> dict:
    """Instructions and block labels of each kernel (comments dropped), from
    its symbol to its end marker (blocks placed after s_endpgm included)."""
    ks, cur = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = ks.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        t = line.split(";")[0].strip()
        if t and (not t.startswith(".") or LABEL.match(t)):
            cur.append(t)
    return ks


def _blocks(lines):
    """Basic blocks (split at labels and after branches) and successors."""
    blocks, cur = [], []
    for t in lines:
        if LABEL.match(t):
            if cur:
                blocks.append(cur)
            cur = [t]
            continue
        cur.append(t)
        if TERMINATOR.match(t):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    where = {b[0][:-1]: i for i, b in enumerate(blocks) if LABEL.match(b[0])}
    succ = []
    for i, b in enumerate(blocks):
        last, s = b[-1], []
        m = re.match(r"^s_branch\s+(\S+)", last)
        if m:
            s = [where[m.group(1)]]
        elif not (last.startswith("s_endpgm") or last.startswith("s_setpc")):
            m = re.match(r"^s_cbranch_\w+\s+(\S+)", last)
            if m:
                s.append(where[m.group(1)])
            if i + 1 < len(blocks):
                s.append(i + 1)
        succ.append(s)
    return blocks, succ


def check_mfma_fences(asm_text: str, where: str, tied=None) -> int:
    """Walk each kernel's control-flow graph with the fact "a matrix
    instruction may have run since the last drain" (the drain: three s_nop 7
    in a row, 24 wait states), and reject an accumulator access (v_accvgpr_*)
    while the fact holds:
      * for kernels issuing the hand-tied v_mfma_f32_16x16x32_f16 (whose
        hazards the compiler cannot see; `tied` None: decided per kernel by
        the presence of that instruction): any such access;
      * otherwise (builtin instructions, whose hazards the compiler tracks
        inside a block and along single paths): an access in a block with
        two or more predecessors before any instruction of its own, the
        case in which this compiler was seen to omit the wait states.
    Also requires wait states (an s_nop) between the last accumulator write
    and the first instruction on the straight-line prologue.  Returns the
    number of kernels checked; raises RuntimeError naming each violation."""
    bad, checked = [], 0
    for name, lines in _kernels(asm_text).items():
        k_tied = any(t.startswith(TIED_MFMA) for t in lines) if tied is None else tied
        mfma = TIED_MFMA if k_tied else "v_mfma_"
        idx = [i for i, t in enumerate(lines) if t.startswith(mfma)]
        if not idx:
            continue
        checked += 1
        head = lines[:idx[0]]
        w = max((i for i, t in enumerate(head) if ACC_ACCESS.match(t)), default=-1)
        if w >= 0 and not any(t.startswith("s_nop") for t in head[w + 1:]):
            bad.append(f"{name}: no wait states between the zero fill and the first instruction")
        blocks, succ = _blocks(lines)
        npred = [0] * len(blocks)
        for s in succ:
            for t in s:
                npred[t] += 1

        def walk(i, live, report):
            ran, nops = False, 0
            for t in blocks[i]:
                if t.startswith(mfma):
                    live, ran, nops = True, True, 0
                    continue
                if t.startswith("s_nop 7"):
                    nops += 1
                    live = live and nops < 3
                    continue
                nops = 0
                if live and ACC_ACCESS.match(t) and (k_tied or (not ran and npred[i] >= 2)):
                    if report:
                        bad.append(f"{name}: accumulator access while a matrix instruction "
                                   f"may be in flight: {t}")
                        return live
            return live

        live_in = [False] * len(blocks)
        changed = True
        while changed:
            changed = False
            for i in range(len(blocks)):
                if walk(i, live_in[i], False):
                    for t in succ[i]:
                        if not live_in[t]:
                            live_in[t] = changed = True
        for i in range(len(blocks)):
            walk(i, live_in[i], True)
    if bad:
        raise RuntimeError(f"matrix-instruction check failed in {where}:\n" + "\n".join(bad))
    return checked


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    checked = src in CHECKED_SOURCES
    extra = ["-save-temps=obj"] if checked else []   # keeps the device assembly in OBJDIR
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if checked:
        stem = os.path.splitext(os.path.basename(src))[0]
        asm = os.path.join(OBJDIR, f"{stem}-hip-amdgcn-amd-amdhsa-gfx950.s")
        with open(asm) as f:
            text = f.read()
        if check_mfma_fences(text, src) == 0:
            raise RuntimeError(f"{src}: no kernel issues a matrix instruction")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
