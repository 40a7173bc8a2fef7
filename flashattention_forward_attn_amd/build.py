"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m flashattention_forward_attn_amd.build``.  Objects go to
``_build/`` beside this file; the library is written next to this file, where
the binding loads it.  A second library, libfa_single_stage.so, differs only in
the forward kernels, compiled with FA_SINGLE_STAGE=1 (one LDS stage, no load in
flight while a tile is read); tests require its results to equal libfa.so's bit
for bit.  Nothing but those tests loads it.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libfa.so")
SINGLE_STAGE_LIBRARY = os.path.join(HERE, "libfa_single_stage.so")
SINGLE_STAGE_SOURCES = ("fa_fwd_bf16.hip", "fa_fwd_fp8.hip")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, single_stage: bool = False) -> str:
    sub = os.path.join(BUILD_DIR, "single_stage") if single_stage else BUILD_DIR
    os.makedirs(sub, exist_ok=True)
    obj = os.path.join(sub, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DFA_SINGLE_STAGE=1"] if single_stage else []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, library: str) -> None:
    tmp = library + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, library)


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa.so and libfa_single_stage.so.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    single = [s for s in srcs if os.path.basename(s) in SINGLE_STAGE_SOURCES]
    assert len(single) == len(SINGLE_STAGE_SOURCES), "single-stage sources missing"
    jobs = [(s, False) for s in srcs] + [(s, True) for s in single]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        objs = list(pool.map(lambda j: _compile(*j), jobs))
    main = objs[:len(srcs)]
    _link(main, LIBRARY)
    swap = {os.path.basename(o): o for o in objs[len(srcs):]}
    _link([swap.get(os.path.basename(o), o) for o in main], SINGLE_STAGE_LIBRARY)
    if verbose:
        print(f"built {LIBRARY} from {len(srcs)} sources and {SINGLE_STAGE_LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
