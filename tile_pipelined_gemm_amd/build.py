"""Builds libmk.so (all HIP sources for gfx950) in-tree.

Usage: python -m tile_pipelined_gemm_amd.build   (or build() from Python)
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

try:
    from . import isa_check
except ImportError:                      # run as a script
    import isa_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_host.hip", "mk_ag_gemm.hip", "mk_gemm_rs.hip", "mk_moe.hip", "mk_moe_combine.hip", "mk_ring_attn.hip",
           "mk_moe_gate.hip", "mk_peak.hip", "mk_litmus.hip"]
ARCH = "gfx950"


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # Packed fp32 instructions stay off (the compiler would otherwise
            # form them from ordinary float code).
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(os.path.dirname(HERE), "include")]


def device_asm(src):
    """Path of the gfx950 assembly the compile of src leaves in _build."""
    return os.path.join(BUILD, f"{os.path.splitext(src)[0]}-hip-amdgcn-amd-amdhsa-{ARCH}.s")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    # -save-temps=obj keeps the device assembly next to the object for the
    # barrier-loop check below
    cmd = [hipcc(), *flags(), "-save-temps=obj", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    found = isa_check.check_file(device_asm(src))
    if found:
        lines = [f"  {k}: {v[:3]}" for k, v in found.items()]
        raise RuntimeError(f"{src}: barrier loop with a per-lane exit (kernel could spin for ever), "
                           "register spills inside an MFMA loop, a wide store whose data is "
                           "rewritten right after it, or an LDS DMA right after an M0 write:\n" + "\n".join(lines))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
