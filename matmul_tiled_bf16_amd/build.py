"""Build libtgemm.so (gfx950) from csrc/ with hipcc, in-tree.

The kernel instances are split over one object per (input type, output type,
trans_a, trans_b) so that they compile in parallel.  The exact compiler
command lines are written to _build/compile_commands.txt.

    python -m matmul_tiled_bf16_amd.build          # incremental
    python -m matmul_tiled_bf16_amd.build --force  # rebuild everything
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Release build for gfx950 only.  Packed fp32 instructions are disabled: hipcc
# must not emit v_pk_{add,mul,fma}_f32.
FLAGS = ["-O3", "-DNDEBUG", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]

TYPES = {"bf16": "__bf16", "f16": "_Float16", "f32": "float"}
IO = [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")]


def _units():
    units = [("tgemm", os.path.join(CSRC, "tgemm.hip"), []),
             ("inst_skinny", os.path.join(CSRC, "inst_skinny.hip"), []),
             ("attention", os.path.join(CSRC, "attention.hip"), []),
             ("splitk", os.path.join(CSRC, "splitk.hip"), [])]
    for i, o in IO:
        for ta in (0, 1):
            for tb in (0, 1):
                tag = f"{i}_{o}_{ta}{tb}"
                defs = [f"-DTG_IN={TYPES[i]}", f"-DTG_OUT={TYPES[o]}", f"-DTG_TA={ta}", f"-DTG_TB={tb}",
                        f"-DTG_TABLE_TILE=tile_{tag}", f"-DTG_TABLE_GENERIC=generic_{tag}",
                        f"-DTG_TABLE_GROUP=group_{tag}"]
                units.append((f"inst_tile_{tag}", os.path.join(CSRC, "inst_tile.hip"), defs))
    return units


def _stale(obj: str, src: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [src] + glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(HERE, "..", "include", "tgemm.h")]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


def build(force: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for name, src, defs in _units():
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        cmd = [HIPCC] + FLAGS + defs + ["-c", src, "-o", obj]
        cmds.append(cmd)
        if force or _stale(obj, src):
            cmds[-1] = (cmd, True)
        else:
            cmds[-1] = (cmd, False)
    todo = [c for c, need in cmds if need]
    jobs = jobs or min(16, os.cpu_count() or 8)

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed:\n{shlex.join(cmd)}\n{r.stderr[-4000:]}")
        if verbose:
            print(shlex.join(cmd[-3:]), flush=True)

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(run, todo))
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", LIB + ".tmp"] + objs
    if todo or not os.path.exists(LIB):
        subprocess.run(link, check=True)
        os.replace(LIB + ".tmp", LIB)
    with open(os.path.join(BUILD, "compile_commands.txt"), "w") as f:
        for c, _ in cmds:
            f.write(shlex.join(c) + "\n")
        f.write(shlex.join(link) + "\n")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    print(build(force=a.force, jobs=a.jobs, verbose=True))


if __name__ == "__main__":
    sys.exit(main())
