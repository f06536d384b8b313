"""Build libra.so (the HIP kernels and the C ABI of include/ra.h) for gfx950.

The library is compiled in-tree with hipcc so it travels with the source tree:
``python -m blockwise_online_softmax_fold_amd.build``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libra.so")
# the plain-C example client of the ABI (tests/c/ring_forward_c.c), built beside libra.so
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "ring_forward_c.c")
C_CLIENT_PATH = os.path.join(PKG_DIR, "ring_forward_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = ["ra_api.hip", "fold_bf16.hip", "fold_f32.hip", "fold_bwd_bf16.hip", "fold_bwd_f32.hip", "state.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def build_command(out_path: str, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fvisibility=hidden",
        # no packed-fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE,
        "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out_path,
        *(extra or []),
    ]


def c_client_command(out_path: str, lib_dir: str = PKG_DIR) -> list[str]:
    """gcc command for the plain-C client, linked against libra.so in lib_dir."""
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    return [
        cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
        "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
        C_CLIENT_SRC, "-o", out_path,
        "-L", lib_dir, "-l:libra.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
        f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
    ]


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain-C client against the in-tree libra.so."""
    cmd = c_client_command(C_CLIENT_PATH)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    return C_CLIENT_PATH


def build(verbose: bool = False) -> str:
    """Compile libra.so (always recompiles) and the C client.  Returns the library path."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_c_client(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
