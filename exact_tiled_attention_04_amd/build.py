"""Build the HIP library libeta_attn.so for gfx950 in-tree.

    python -m exact_tiled_attention_04_amd.build [--resource-usage]

Each source is compiled to an object in parallel with hipcc, then linked
into ``exact_tiled_attention_04_amd/libeta_attn.so``.  Packed-fp32 VALU
instructions are disabled for all device code.  ``--resource-usage`` prints
the compiler's per-kernel register, LDS and scratch report.
"""

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libeta_attn.so")
SOURCES = ["api.hip", "fwd.hip", "decode.hip", "bwd.hip"]
ARCH = "gfx950"


def _hipcc():
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build")


def compile_flags(resource_usage=False):
    flags = [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-munsafe-fp-atomics",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
    ]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    return flags


def build(verbose=False, resource_usage=False, jobs=None):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    flags = compile_flags(resource_usage)

    def one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        return obj, res.stderr

    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(one, SOURCES))
    if verbose or resource_usage:
        for (_, err), src in zip(results, SOURCES):
            lines = [ln for ln in err.splitlines()
                     if resource_usage and "remark" in ln or (verbose and "error" in ln)]
            if lines:
                print(f"== {src}")
                print("\n".join(lines))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[obj for obj, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    build(verbose=True, resource_usage=args.resource_usage)
    return 0


if __name__ == "__main__":
    sys.exit(main())
