"""Build libmsda.so (the C-ABI library and its gfx950 kernels) and
libmsda_micro.so (the measurement kernels of include/msda_micro.h) in-tree
with hipcc.

    python -m scale_deformable_attention_03_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsda.so")
# the C ABI and one translation unit of kernel instantiations per dtype code,
# compiled in parallel and linked into one library
SOURCES = [os.path.join(CSRC, f) for f in ("msda_api.hip", "msda_kernels_f32.hip", "msda_kernels_f16.hip",
                                            "msda_kernels_bf16.hip", "msda_kernels_f16_f32.hip",
                                            "msda_kernels_bf16_f32.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("msda_types.hpp", "msda_plan.hpp", "msda_device.hpp", "msda_forward.hpp", "msda_backward.hpp",
                                           "msda_launch.hpp", "msda_launch_impl.hpp")] + [os.path.join(INCLUDE, "msda.h")]
MICRO_LIB = os.path.join(PKG, "libmsda_micro.so")
MICRO_SOURCES = [os.path.join(CSRC, "msda_micro.hip")]
MICRO_HEADERS = [os.path.join(INCLUDE, "msda_micro.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Wall", "-Wno-unused-result", "-Wno-pass-failed",
    # float32 atomics compile to the hardware global_atomic_add_f32
    "-munsafe-fp-atomics",
    # no packed-fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    """Compile every source (always recompiles): one hipcc process per
    source, all in parallel, then one link per library.  Returns the path of
    libmsda.so."""
    targets = [(LIB, SOURCES), (MICRO_LIB, MICRO_SOURCES)]
    procs, objs = [], {}
    for lib, sources in targets:
        for src in sources:
            obj = os.path.join(CSRC, os.path.basename(src)[:-4] + ".o")
            cmd = [HIPCC, *FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd), cmd))
            objs.setdefault(lib, []).append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    for lib, _ in targets:
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib + ".tmp", *objs[lib]]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(lib + ".tmp", lib)
        for obj in objs[lib]:
            os.remove(obj)
    return LIB


def stale() -> bool:
    """True when the library is missing or older than a source or header."""
    for lib, deps in ((LIB, SOURCES + HEADERS), (MICRO_LIB, MICRO_SOURCES + MICRO_HEADERS)):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        if any(os.path.getmtime(f) > t for f in deps):
            return True
    return False


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
