"""Build libnanoflow.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP and C++ source under csrc/ is compiled to an object under _build/ at the repo
root (in parallel), then linked into nano_intra_overlap_amd/libnanoflow.so. Run as
``python -m nano_intra_overlap_amd.build``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnanoflow.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed-fp32 instructions stay off: hipcc -O3 forms v_pk_* from ordinary float code
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-Wno-unused-but-set-variable", f"-I{os.path.join(ROOT, 'include')}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
# attention: MFMA accumulators in ordinary VGPRs (fewer registers, no AGPR copies around the
# online-softmax rescale), which leaves room for GEMM waves on the same SIMD
PER_FILE_FLAGS = {"nf_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                  "nf_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *COMMON, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
