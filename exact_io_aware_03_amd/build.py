"""Build libfa.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m exact_io_aware_03_amd.build [--jobs N] [--debug] [--sched-strategy NAME]

Every source under csrc/ is compiled for gfx950 with packed-fp32 instruction selection
disabled and without type-based alias analysis (the kernels reuse LDS areas through pointers of
several types), then linked into exact_io_aware_03_amd/libfa.so next to this file.

--sched-strategy builds with one of LLVM's other AMDGPU machine-scheduler strategies (max-ilp,
max-memory-clause, iterative-ilp, iterative-minreg) into libfa_<strategy>.so instead; the
binding loads it when FA_LIB_VARIANT=<strategy> is set. Running the GPU tests against such a
build checks that no kernel depends on an instruction order the compiler is free to change (a
missing wait or fence). libfa.so is never replaced by such a build, and fa_build_info() names
the strategy a library was built with.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}",
    "-std=c++17",
    "-fPIC",
    "-Wno-unused-result",
    "-Werror=array-bounds",
    # LDS areas are reused through pointers of several types (fp32 partials, bf16 pairs, 16-byte
    # rows): type-based alias analysis must not reorder those accesses
    "-fno-strict-aliasing",
    # keep the compiler from forming v_pk_{add,mul,fma}_f32 (host pass warns it does not know it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fp8.hip", "fa_decode.hip", "fa_bwd.hip"]


def _compile(src: str, opt: list[str], obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *opt, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(jobs: int = 4, debug: bool = False, verbose: bool = True, sched_strategy: str | None = None) -> str:
    obj_dir = OBJ_DIR + (f"_{sched_strategy}" if sched_strategy else "")
    out = os.path.join(HERE, f"libfa_{sched_strategy}.so") if sched_strategy else OUT
    os.makedirs(obj_dir, exist_ok=True)
    opt = ["-O1", "-g"] if debug else ["-O3"]
    info = f"{ARCH} {'-O1 -g' if debug else '-O3'} sched={sched_strategy or 'default'}"
    opt += [f'-DFA_BUILD_INFO="{info}"']
    if sched_strategy:
        opt += ["-mllvm", f"-amdgpu-sched-strategy={sched_strategy}"]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, opt, obj_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} ({info})")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--sched-strategy", choices=["max-ilp", "max-memory-clause", "iterative-ilp", "iterative-minreg"])
    args = ap.parse_args()
    try:
        build(args.jobs, args.debug, sched_strategy=args.sched_strategy)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
