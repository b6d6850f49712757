"""Build libmtb.so for gfx950 with hipcc (in-tree, next to this file).

    python -m transformer_layer_ln_amd.build

Regenerates ``csrc/gemm_loop.inc``, compiles every ``csrc/*.hip`` to an object in ``_build/`` (in parallel) and
links the shared library. Always recompiles: it is the "does it build" check.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmtb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# per-source additions: the cross-entropy kernels are arithmetic-bound on their
# max reductions and exponentials; without IEEE mode a float max needs no
# input canonicalisation (logits are finite)
FILE_FLAGS = {"xent.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # the GEMM main loop is generated (csrc/gen_gemm_loop.py -> csrc/gemm_loop.inc)
    rc, out = _run([sys.executable, os.path.join(CSRC, "gen_gemm_loop.py")])
    if rc != 0:
        print(out)
        raise RuntimeError("libmtb: generating gemm_loop.inc failed")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            print(" ".join(cmd))
            if out:
                print(out)
        failed |= rc != 0
    if failed:
        raise RuntimeError("libmtb: compilation failed")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out)
        raise RuntimeError("libmtb: link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
