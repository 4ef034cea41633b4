"""Builds libmoe_ep.so in-tree with hipcc for gfx950 (MI355X), and beside it
libmoe_ceilings.so, the pattern-ceiling kernels the benchmark times.

Each HIP source is compiled to an object in parallel, then linked into its
shared library next to this file.  Flags:
  -ffp-contract=off            no implicit fused multiply-adds: combine's fma
                               chain is spelled out, nothing else is fused
  -target-feature -packed-fp32-ops
                               keep the compiler from forming packed fp32 ops
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_ep.so")
SOURCES = ["api.hip", "layout.hip", "dispatch.hip", "combine.hip", "fused.hip", "balance.hip", "padding.hip"]
CEIL_LIB = os.path.join(HERE, "libmoe_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _build_lib(lib: str, sources, verbose: bool) -> str:
    with tempfile.TemporaryDirectory(prefix="moe_ep_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l and l.strip())
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if verbose and out:
                print(out)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(sources)) as ex:
            objs = list(ex.map(compile_one, sources))
        tmp_lib = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp_lib, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe_ep.so and
    libmoe_ceilings.so (always rebuilds).  Returns the path of libmoe_ep.so."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=2) as ex:
        main = ex.submit(_build_lib, LIB, SOURCES, verbose)
        ceil = ex.submit(_build_lib, CEIL_LIB, CEIL_SOURCES, verbose)
        ceil.result()
        return main.result()


if __name__ == "__main__":
    print(build(verbose=True))
