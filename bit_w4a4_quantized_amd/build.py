"""Build libsvdq.so (gfx950) in-tree with hipcc.

    python -m bit_w4a4_quantized_amd.build        # or build() from Python

All HIP sources are compiled for gfx950 only.  Packed-fp32 VALU instructions
are disabled (-packed-fp32-ops): the compiler would otherwise form them from
scalar float code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvdq.so")
SOURCES = ["svdq_api.hip", "k_quant_down.hip", "k_quant_weight.hip", "k_gemm.hip", "k_gemm2.hip",
           "k_gemm3.hip", "k_gemm_i8.hip", "k_gemm_f4.hip", "k_gemm_mx.hip", "k_w4a16.hip", "k_misc.hip", "k_relayout.hip"]
# -amdgpu-mfma-vgpr-form: MFMA results in VGPRs, so the per-group rescale reads
# them without v_accvgpr_read copies.  Not for the MXFP4 GEMM, whose four-wave kernel keeps
# 256 accumulators per lane in the accumulation registers (its other kernels come out the same
# either way).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-result"]
AGPR_SOURCES = {"k_gemm_mx.hip"}


def source_flags(src: str) -> list:
    if src not in AGPR_SOURCES:
        return FLAGS
    return [f for i, f in enumerate(FLAGS) if f != "-amdgpu-mfma-vgpr-form" and
            not (f == "-mllvm" and i + 1 < len(FLAGS) and FLAGS[i + 1] == "-amdgpu-mfma-vgpr-form")]
BUILD_DIR = os.path.join(HERE, "_build")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libsvdq.so.  Always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *source_flags(src), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


# The C ABI's host code (argument validation, workspace carving) built with AddressSanitizer
# and UndefinedBehaviorSanitizer for the host pass only (each -fsanitize after -Xarch_host), linked
# with tests/abi_check.cpp: a program that drives every validation path without a GPU.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
HOST_CHECK = os.path.join(BUILD_DIR, "svdq_abi_check")


def build_host_check(verbose: bool = False) -> str:
    """Compile svdq_api.hip with the sanitizers (the other objects come from build()) and link
    the ABI check program; returns its path."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, s.replace(".hip", ".o"))) for s in SOURCES):
        build(verbose)
    cc = hipcc()
    api = os.path.join(BUILD_DIR, "svdq_api_sanitized.o")
    _run([cc, *FLAGS, *SANITIZE, "-c", os.path.join(CSRC, "svdq_api.hip"), "-o", api], verbose)
    objs = [api] + [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "svdq_api.hip"]
    check = os.path.join(os.path.dirname(HERE), "tests", "abi_check.cpp")
    _run([cc, "--offload-arch=gfx950", *SANITIZE, "-x", "c++", check, "-x", "none", *objs, "-o", HOST_CHECK],
         verbose)
    return HOST_CHECK


MICROBENCH = os.path.join(BUILD_DIR, "mfma_valu")


def build_microbench(verbose: bool = False) -> str:
    """The microbenchmarks, programs of their own (not part of the library): matrix-core /
    vector-ALU overlap (microbench/mfma_valu.hip), the operand load paths
    (microbench/load_paths.hip), the sustained matrix-core rates with the clock they hold
    (microbench/mfma_clock.hip) and the weight stream of the few-token-rows kernel
    (microbench/weight_stream.hip).  Returns the first program's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    # mfma_valu without the VGPR-form flag: its AGPR cases need the compiler free to put MFMA
    # results in AGPRs (the others get the VGPR form either way)
    no_vgpr_form = source_flags("k_gemm_mx.hip")
    _run([hipcc(), *no_vgpr_form, os.path.join(HERE, "microbench", "mfma_valu.hip"), "-o", MICROBENCH], verbose)
    for prog in ("load_paths", "mfma_clock", "weight_stream"):
        _run([hipcc(), *FLAGS, os.path.join(HERE, "microbench", prog + ".hip"), "-o", os.path.join(BUILD_DIR, prog)],
             verbose)
    return MICROBENCH


if __name__ == "__main__":
    if "--microbench" in sys.argv:
        print(build_microbench(verbose="-v" in sys.argv))
    elif "--host-check" in sys.argv:
        print(build_host_check(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
