"""Build libqsa.so (gfx950) in-tree with hipcc.

    python -m block_sparse_trainable_amd.build [--verbose]

Every source under csrc/ is compiled to an object (in parallel), then linked
into block_sparse_trainable_amd/libqsa.so next to this file.  hipcc
cross-compiles for gfx950 without a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libqsa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags.  The scoring kernels keep their MFMA accumulators in
# ordinary VGPRs: the epilogue reads every accumulator, and AGPR-held ones
# would each cost a copy instruction.
EXTRA = {
    "score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # no NaN reaches the distillation kernels' max and exponent chains (masked
    # logits are -inf, still honoured): without this each fmaxf of an MFMA
    # result first quiets its operand, a VALU instruction per score
    "distill.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizers for the C-ABI layer: AddressSanitizer and UBSan on the
# host pass only (device code is never instrumented), UB fatal.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime the sanitized library links to
    (to be preloaded into an uninstrumented host process)."""
    res = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build_sanitized(out: str) -> str:
    """libqsa with the C-ABI source (qsa_api.hip: validation, workspace sizes,
    dispatch) compiled with host ASan + UBSan, linked with the ordinary
    objects of the kernel sources, into `out`."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    for src in sources():
        if os.path.basename(src) == "qsa_api.hip":
            obj = os.path.join(OBJDIR, "qsa_api.san.o")
            cmd = [HIPCC, *CFLAGS, *SAN_HOST, "-c", src, "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}{res.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
                obj = _compile(src, False)
            objs.append(obj)
    # host link (the device code is already embedded in each object)
    cmd = [CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", out, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stdout}{res.stderr}")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true", help="print kernel resource usage")
    a = ap.parse_args(argv)
    print(build(a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
