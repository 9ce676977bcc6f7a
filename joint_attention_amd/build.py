"""Build libjoint_attn.so (gfx950) in-tree with hipcc.

    python -m joint_attention_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops) and fast-math off; the shared object lands next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libjoint_attn.so")
ARCH = os.environ.get("JA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["joint_attn.cpp", "pack.hip", "fwd_bf16.hip", "quant_fp8.hip", "fwd_fp8.hip"]

# per-source code-generation options: the bf16 forward keeps its MFMA accumulators in
# architectural VGPRs (the score tiles are read by the softmax right away), which is
# what lets its 32-row output accumulators, two score tiles, two P tiles and the staged
# K/V tiles fit in 256 VGPRs without spilling at two waves per SIMD
# (and, no NaN ever being an operand there, skips the NaN canonicalisation in front of
# every v_max; infinities keep their meaning)
EXTRA_FLAGS = {"fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
               "fwd_fp8.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def compile_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-fast-math", "-ffp-contract=fast",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I" + INCLUDE, "-I" + CSRC]


def build(verbose: bool = False, jobs: int = 8, out: str | None = None,
          defines: tuple = ()) -> str:
    """Compile every source to an object (in parallel), link the shared library
    (to `out`, default libjoint_attn.so here; `defines` adds -D options)."""
    lib_path = out or LIB
    objdir = os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build",
                          os.path.basename(lib_path).replace(".so", ""))
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = ([hipcc()] + compile_flags() + ["-D" + d for d in defines] +
               EXTRA_FLAGS.get(src, []) + lang +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the gfx-only feature flag; that warning is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "-v"]
    out = next((a[len("--out="):] for a in args if a.startswith("--out=")), None)
    defs = tuple(a[2:] for a in args if a.startswith("-D"))
    print(build(verbose="-v" in sys.argv, out=out, defines=defs))
