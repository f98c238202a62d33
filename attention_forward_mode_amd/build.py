"""Build libattn_jvp.so in-tree: HIP kernels for gfx950 plus the C ABI; and
libmfma_probe.so, the matrix-core throughput probe the benchmark reports
beside the published peak (include/mfma_probe.h).

    python -m attention_forward_mode_amd.build        # or __graft_entry__.build()

hipcc cross-compiles gfx950 code objects without a GPU.  Every HIP source is
compiled with packed-fp32 instructions disabled (the compiler would otherwise
form v_pk_* fp32 ops on its own); hipcc's host pass warns that it does not know
that feature, which is harmless.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn_jvp.so")
PROBE_LIB = os.path.join(PKG, "libmfma_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["attn_jvp_bf16.hip", "attn_jvp_f32.hip", "attn_jvp_merge.hip", "attn_bwd.hip",
               "attn_jvp_noalloc.hip"]
CXX_SOURCES = ["attn_jvp_api.cpp"]
PROBE_SOURCE = "mfma_probe.hip"

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fvisibility=hidden", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, save_temps=False):
    """Compile every source and link libattn_jvp.so and libmfma_probe.so;
    always rebuilds."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        extra = ["-save-temps=obj"] if save_temps else []
        _run([hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lamdhip64"], verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64"], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
    print(LIB)
