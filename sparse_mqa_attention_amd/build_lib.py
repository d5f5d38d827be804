"""Build libdsa.so (the HIP kernels and the C ABI) in place with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["abi.cpp", "index_scores.hip", "index_scores_prefill.hip", "index_scores_mxfp4.hip", "topk.hip", "sparse_attn.hip", "sparse_attn_decode.hip",
           "sparse_attn_prefill.hip", "sparse_attn_f32.hip", "noalloc.hip",
           "epilogue.hip"]
ARCH = "gfx950"
# packed fp32 VALU forms are kept out of the generated code
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]
# per-source additions: the prefill index kernel's MFMA accumulators feed VALU work every tile
# (its epilogue rectifies and weights them), so they stay in VGPRs rather than AGPRs that would be
# copied out first
EXTRA_FLAGS = {"index_scores_prefill.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source and link libdsa.so next to this file; returns its path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
