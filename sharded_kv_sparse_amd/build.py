"""Build libdcpmla.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m sharded_kv_sparse_amd.build [--verbose]
Writes sharded_kv_sparse_amd/libdcpmla.so.  Compiles every time it is run.
"""

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdcpmla.so")
SOURCES = ["dcp_api.cpp", "dcp_remap.hip", "dcp_combine.hip", "dcp_decode.hip",
           "dcp_decode_fp8.hip", "dcp_kv_write.hip", "dcp_noalloc.hip",
           "dcp_prefix.hip", "dcp_index_topk.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-lambda-capture",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in architectural VGPRs: the online-softmax rescale of
    # O is then a plain VALU multiply instead of AGPR<->VGPR round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose=False, jobs=4):
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="dcpmla_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc] + HIPCC_FLAGS + ["-c"] + lang + [os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = out.decode(errors="replace")
            lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
            if pr.returncode != 0:
                failed.append(src)
                print("\n".join(lines), file=sys.stderr)
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError("hipcc failed for " + ", ".join(failed))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
