"""Build libpkv.so (the HIP kernels + C-ABI) in-tree for gfx950 with hipcc.

Usage: python -m paged_kv_cache_288_amd.build [--isa]
  --isa  also keep the device assembly (.s) of every source under _build/ for inspection.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
READ_CEILING = os.path.join(HERE, "read_ceiling")   # standalone bandwidth probe
ARCH = "gfx950"

SOURCES = ["pkv_api.hip", "kv_append.hip", "gqa_decode.hip", "gqa_stream.hip", "mla_decode.hip",
           "mla_stream.hip", "gqa_multi.hip", "gqa_cascade.hip", "validate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # Keep the compiler from forming packed fp32 ops (v_pk_fma_f32 and friends).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The latent balanced kernel keeps its MFMA accumulators in VGPRs:
# in AGPRs the compiler copies them around the kernel's rare rescale branch at every stage.
# The multi-token kernel's 64-row variant needs the same to stay out of scratch.
SOURCE_FLAGS = {"mla_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gqa_multi.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gqa_cascade.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, isa):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if isa:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    # The host pass does not know the device-only feature above; drop that warning.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(isa=False, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, isa), SOURCES))
    for (obj, err) in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    for exe in (READ_CEILING,):
        src = os.path.basename(exe) + ".hip"
        cmd = [HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", exe + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        os.replace(exe + ".tmp", exe)
    if verbose:
        print(f"built {LIB} and {READ_CEILING}")
    return LIB


if __name__ == "__main__":
    build(isa="--isa" in sys.argv)
