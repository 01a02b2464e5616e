"""Build libring_attn.so (the C-ABI ring-attention library) for gfx950 in-tree.

    python -m ring_attention_step_amd.build

Every HIP source is compiled with hipcc for gfx950 only; packed-fp32 VALU
instructions are disabled (-packed-fp32-ops), the host-only planner is
compiled as ordinary C++.  The result lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libring_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
HIP_SOURCES = ["api.hip", "step_bf16.hip", "ring_fwd.hip", "step_f32.hip", "finalize_merge.hip", "pack_vt.hip",
               "key_bits.hip", "backward.hip"]
# Per-file code generation options.  ring_fwd.hip keeps its score accumulators
# in VGPRs (the vector ALU reads them) and its Q operands in AGPRs: the VGPR
# form of the matrix instructions.
EXTRA_FLAGS = {"ring_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CPP_SOURCES = ["plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def _common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall"]


def build(verbose: bool = False) -> str:
    tmpdir = tempfile.mkdtemp(prefix="ring_attn_build_")
    try:
        cmds = []
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            objs.append(obj)
            cmds.append([hipcc(), "-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
                         "-packed-fp32-ops", "-munsafe-fp-atomics", *EXTRA_FLAGS.get(src, []), *_common_flags(), "-c",
                         os.path.join(CSRC, src), "-o", obj])
        for src in CPP_SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            objs.append(obj)
            cmds.append(["g++", *_common_flags(), "-c", os.path.join(CSRC, src), "-o", obj])

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            # hipcc's host pass does not know the device-only feature name.
            err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
            if r.returncode != 0:
                raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
            if err.strip() and verbose:
                print(err)

        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            list(ex.map(run, cmds))
        tmp_lib = os.path.join(tmpdir, LIB_NAME)
        link = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp_lib]
        run(link)
        os.replace(tmp_lib, LIB_PATH) if os.path.dirname(tmp_lib) == HERE else shutil.move(tmp_lib, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
