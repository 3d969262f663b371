"""Build libgsa.so (all HIP kernels + the C ABI) in-tree with hipcc for gfx950.

Usage:  python -m gated_softmax_attention_amd.build
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libgsa.so")
SOURCES = ["api.hip", "gate_gemm.hip", "attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip", "gemm_bwd.hip", "attn_diag.hip", "value_gate.hip", "gate_shared.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False, out: str = LIB_PATH, csrc: str = CSRC, extra=()) -> str:
    """Compile every source into libgsa.so (next to this file by default); return its path."""
    srcs = [os.path.join(csrc, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=PKG, prefix=".libgsa.")
    os.close(fd)
    cmd = [HIPCC, "-I", csrc] + FLAGS + list(extra) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
        if verbose and res.stderr:
            # hipcc's host pass warns about the gfx-only target feature; keep other lines
            lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
            if lines:
                print("\n".join(lines[-40:]), file=sys.stderr)
        shutil.move(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out


def ensure_built(verbose: bool = False) -> str:
    """The tests, the smoke check and the bench load the library that is built;
    only when none is there do they build it first.  (The binding itself never
    builds: without libgsa.so it raises.)"""
    if not os.path.exists(LIB_PATH):
        build(verbose=verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
