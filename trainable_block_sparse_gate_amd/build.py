"""Build ``libsas.so`` (the HIP kernels + C ABI) for gfx950 with hipcc.

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so the binding finds it in-tree.  The same call
builds ``libsas_peaks.so`` (``csrc/peaks.hip``), the MFMA-loop and
streaming-read kernels the benchmark measures the device's peaks with; the
SAS library does not contain or load it.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsas.so")
PEAKS_LIB = os.path.join(HERE, "libsas_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sas_api.cpp", "gate.hip", "fwd.hip", "bwd.hip", "bwd_dkdv.hip", "decode.hip"]
PEAKS_SOURCES = ["peaks.hip"]

# Kernels whose accumulators and MFMA results are better placed by asking for
# the VGPR form of MFMA (fewer accumulator moves between AGPRs and VGPRs in the
# inner loop; measured faster for these two, slower for the dq kernel).
MFMA_VGPR_FORM = {"fwd.hip", "bwd_dkdv.hip"}

# Packed fp32 VALU ops are kept off: hipcc would otherwise form them from
# ordinary float code.
COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, "-c"]
    if src in MFMA_VGPR_FORM:
        cmd += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += [path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def _link(objs, out, verbose):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES + PEAKS_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES if s in objs], LIB, verbose)
    _link([objs[s] for s in PEAKS_SOURCES if s in objs], PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
