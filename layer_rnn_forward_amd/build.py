"""Build ``librnn_mi355x.so`` (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: ``python -m layer_rnn_forward_amd.build`` or ``build()`` from Python.
Compiles every source each time it is called.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librnn_mi355x.so")
SOURCES = ["dropout.hip", "gemm.hip", "layout.hip", "recurrent.hip", "recurrent_gru2.hip", "rnn_api.cpp",
           *[f"recurrent_{m}_{k}.hip" for m in ("tanh", "lstm", "gru") for k in ("fwd", "bwd")]]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# per-source extra flags: the MFMA throughput probes in layout.hip keep their
# accumulators in VGPRs (with AGPR accumulators the compiler rotated some of
# the independent chains through accumulator moves, which halved the
# 16x16x32 bf16 probe's rate)
EXTRA = {"layout.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# host-only sanitizers for the C-ABI translation unit (the planner and its
# workspace carve); device code is built as usual
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_LIB = os.path.join(BUILD, "sanitize", "librnn_mi355x_san.so")
# the ordering-perturbation test build, in-tree beside the library
PERTURB_LIB = os.path.join(PKG, "librnn_mi355x_perturb.so")


def _build(out_lib: str, obj_dir: str, sanitize: bool, verbose: bool, defines=()) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".", "_") + ".o")
        objs.append(obj)
        extra = ["-x", "hip"] if src.endswith(".cpp") else []
        san = SANITIZE if (sanitize and src == "rnn_api.cpp") else []
        cmds.append([HIPCC, *FLAGS, *defines, *EXTRA.get(src, []), *san, *extra, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with ThreadPoolExecutor(max_workers=min(16, len(cmds))) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = out_lib + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] \
        if sanitize else []
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_san, "-o", tmp, *objs])
    os.replace(tmp, out_lib)
    return out_lib


def build(verbose: bool = False) -> str:
    return _build(LIB, BUILD, False, verbose)


def build_perturbed(verbose: bool = False) -> str:
    """The same library with the exchange's ordering points perturbed
    (-DRNN_PERTURB: pseudo-random pauses at every flag wait and flag
    publication); its results must be bitwise those of the normal build.
    Load it with RNN_LIB pointing at the returned path."""
    return _build(PERTURB_LIB, os.path.join(BUILD, "perturb"), False, verbose, defines=("-DRNN_PERTURB",))


def build_sanitized(verbose: bool = False) -> str:
    """The same library with the host code of the C ABI built under
    AddressSanitizer and UndefinedBehaviorSanitizer (run it with the ASan
    runtime preloaded and RNN_LIB pointing at the returned path)."""
    return _build(SAN_LIB, os.path.dirname(SAN_LIB), True, verbose)


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (for LD_PRELOAD)."""
    r = subprocess.run([HIPCC.replace("hipcc", "amdclang++") if os.path.exists(HIPCC.replace("hipcc", "amdclang++"))
                        else HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
