"""Build the gfx950 HIP library libsparse_attn.so in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only.  Packed fp32 vector
instructions are disabled (-packed-fp32-ops) for all device code, and MFMA
instructions use the VGPR form for their accumulators.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["api.cpp", "pool.hip", "route.hip", "fwd_f32.hip", "fwd_bf16.hip", "fwd_bf16_skim.hip", "residual.hip"]
# per-source flags: the skim forms keep their MFMAs beside the softmax work
# only without machine sinking
SOURCE_FLAGS = {"fwd_bf16_skim.hip": ["-mllvm", "-disable-machine-sink"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in VGPRs: the forward kernel's register budget
         # then fits without scratch (AGPRs hold the spare operands)
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, lib_path: str = LIB, defines=(), extra_flags=()) -> str:
    """Compile every source to an object, link libsparse_attn.so; returns its path."""
    build_dir = os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ([HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + list(extra_flags) + [f"-D{x}" for x in defines] + lang
               + ["-c", os.path.join(CSRC, src), "-o", obj])
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for src, cmd, p in procs:
        out = p.communicate()[0].decode()
        out = "\n".join(x for x in out.splitlines() if "packed-fp32-ops" not in x)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
