"""Build libvsa.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m block_sparse_video_cube_amd.build [--jobs N]

Every source under csrc/ is compiled with hipcc for gfx950 and linked into
block_sparse_video_cube_amd/libvsa.so. Compilation always runs (no caching
beyond hipcc's own), so a build after a source change is never stale.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvsa.so")
ARCH = "gfx950"

SOURCES = ["pool.hip", "coarse.hip", "fine_fwd.hip", "fine_bwd.hip", "combine.hip", "backward.hip", "layout.hip",
           "probe.hip", "vsa_api.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the VSA HIP library cannot be built")


# Sources whose kernels issue direct-to-LDS loads through inline assembly that
# sets M0 (fine_common.h). M0 is a register the compiler reserves for its own
# use, so it cannot be declared clobbered; instead every build checks the
# generated gfx950 assembly of these sources (kept by -save-temps) and fails
# if the compiler touches M0 anywhere else in a kernel that issues them.
M0_SOURCES = ("fine_fwd.hip", "fine_bwd.hip")
_DMA = "global_load_lds_dwordx4"
_M0 = re.compile(r"\bm0\b")


def check_m0(asm: str) -> list[str]:
    """Findings in gfx950 assembly text: in every function that issues
    global_load_lds_dwordx4, each instruction naming M0 must be an
    `s_mov_b32 m0, <sgpr>` followed directly by `s_nop 0` and the load, and
    every such load must be preceded by one. Returns the violations."""
    bad = []
    funcs, cur, name = [], [], None
    for line in asm.splitlines():
        code = line.split(";", 1)[0].strip()
        if code.endswith(":") and not code.startswith(".") and " " not in code:
            if name is not None:
                funcs.append((name, cur))
            name, cur = code[:-1], []
            continue
        if code and not code.startswith("."):
            cur.append(code)
    if name is not None:
        funcs.append((name, cur))
    for fname, ins in funcs:
        if not any(i.startswith(_DMA) for i in ins):
            continue
        for n, i in enumerate(ins):
            if i.startswith(_DMA):
                if n < 2 or ins[n - 1] != "s_nop 0" or not re.fullmatch(r"s_mov_b32 m0, \S+", ins[n - 2]):
                    bad.append(f"{fname}: {_DMA} #{n} without its own M0 set-up")
                continue
            if _M0.search(i) is None:
                continue
            if (re.fullmatch(r"s_mov_b32 m0, \S+", i) and n + 2 < len(ins) and ins[n + 1] == "s_nop 0"
                    and ins[n + 2].startswith(_DMA)):
                continue
            bad.append(f"{fname}: M0 used outside the direct-to-LDS loads: {i}")
    return bad


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    temps = ["-save-temps=obj"] if src in M0_SOURCES else []
    cmd = [hipcc(), *FLAGS, *temps, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=OBJ)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    if temps:
        stem = os.path.splitext(os.path.basename(src))[0]
        asm = os.path.join(OBJ, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        with open(asm) as f:
            text = f.read()
        if _DMA not in text:
            raise RuntimeError(f"{src}: no {_DMA} in {asm}; the M0 check saw no loads")
        bad = check_m0(text)
        if bad:
            raise RuntimeError(f"{src}: M0 check failed:\n" + "\n".join(bad[:20]))
    return out


def build(jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    print(build(ap.parse_args().jobs))
