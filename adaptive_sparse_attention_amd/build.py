"""Build libentmax_attn.so for gfx950 with hipcc.

Usage: python -m adaptive_sparse_attention_amd.build [--jobs N]

Every translation unit under csrc/ is compiled to an object in parallel and
linked into ``adaptive_sparse_attention_amd/libentmax_attn.so`` (in-tree).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libentmax_attn.so")
SOURCES = ["api.hip", "k_bf16.hip", "k_f32.hip", "k_mask.hip", "k_peak.hip"]
ARCH = os.environ.get("EA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results straight into arch VGPRs (no AGPR round trips before
        # the elementwise work on score tiles)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-result",
    ]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    return proc.returncode, out


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    cmds = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError(f"link failed\n{out}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
