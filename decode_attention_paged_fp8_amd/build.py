"""Builds libdapf8.so (the HIP library) in-tree with hipcc for gfx950.

Every translation unit is compiled with packed-fp32 instructions disabled and without fast-math
(the quantiser relies on correctly rounded fp32 division), and with matrix-core accumulators kept in
ordinary vector registers.  Object files are compiled in
parallel, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libdapf8.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "kv_ops.hip", "attn_generic.hip", "attn_mfma.hip", "attn_latent.hip", "page_alloc.hip", "w4_gemv.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
            # matrix-core accumulators in ordinary VGPRs: the softmax rescale and the epilogue work on
            # them with vector instructions, and AGPR-resident accumulators cost a copy each window
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(os.path.dirname(HERE), "include")]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="dapf8_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if verbose and out.strip():
                print(out)
            return obj

        with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
