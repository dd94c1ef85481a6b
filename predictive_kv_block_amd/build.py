"""Build libspin.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m predictive_kv_block_amd.build [--jobs N]

Objects go to _build/ at the repository root; the shared library is written
next to this file.  Every call recompiles (hipcc cross-compiles without a GPU).
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspin.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the epilogues read them with plain VALU
    # operands instead of copying each accumulator register out first
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["spin_abi.cpp", "spin_state.hip", "spin_predict.hip", "spin_indexer.hip",
           "spin_topk.hip", "spin_update.hip", "spin_fidelity.hip", "spin_attention.hip"]


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in ln and "ignoring feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs.strip()


def build(jobs=None, verbose=False, out=LIB, build_dir=BUILD, sources=SOURCES):
    """Compile every HIP source and link the library (default: libspin.so next to
    this file)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(sources), os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir), sources))
    for obj, msg in results:
        if msg and verbose:
            print(msg, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results],
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
