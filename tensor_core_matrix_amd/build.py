"""Build libtcm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m tensor_core_matrix_amd.build [--asm DIR] [--sanitize]

Each source is compiled by hipcc in parallel, then linked into
``tensor_core_matrix_amd/libtcm.so``.  ``--asm DIR`` also writes the gfx950
assembly of every kernel source to DIR for inspection.

``--sanitize`` builds ``_build/libtcm_san.so`` instead: the host code (the
C ABI, validation, planning and dispatch in tcm_api.cpp) compiled by g++
with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
ordinary device objects.  It is for CPU runs of the host-side tests, e.g.

    python -m tensor_core_matrix_amd.build --sanitize
    python -c "from oracle import oracle; oracle.build(sanitize=True)"
    LD_PRELOAD=$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    TCM_LIBRARY=_build/libtcm_san.so ORACLE_LIBRARY=oracle/liboracle_san.so \
    python -m pytest tests/test_abi.py tests/test_oracle.py -m "not gpu"
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtcm.so")
SAN_LIB = os.path.join(ROOT, "_build", "libtcm_san.so")
# host-only sanitizer flags (g++; the device code is built as usual)
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]
ARCH = "gfx950"
SOURCES = ["tcm_api.cpp", "gemm_tn.hip", "gemm_mx.hip", "gemm_mx6.hip", "gemm_nv4.hip", "gemm_epi.hip",
           "gemm_mn_a.hip", "gemm_mn_b.hip", "gemm_mn_ab.hip", "gemm_mx_ld.hip", "gemm_mx_mn_a.hip",
           "gemm_mx_mn_b.hip", "gemm_mx_mn_ab.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
# Packed fp32 VALU forms are kept out of the device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast", "-munsafe-fp-atomics"]


def _compile(src: str, asm_dir: str | None, sanitize: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + (".san.o" if sanitize else ".o"))
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:  # host-only C++: the C ABI, validation and dispatch
        cmd = ["g++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", *COMMON,
               *(SANITIZE if sanitize else []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if err.strip():
        print(err, file=sys.stderr)
    if r.returncode:
        raise RuntimeError(f"compile failed: {src}")
    if asm_dir and src.endswith(".hip"):
        out = os.path.join(asm_dir, src + ".s")
        subprocess.run([HIPCC, "-x", "hip", *DEVICE, *COMMON, "--cuda-device-only", "-S", path,
                        "-o", out], check=True, stderr=subprocess.DEVNULL)
    return obj


def build(asm_dir: str | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
                    "-lamdhip64"], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """_build/libtcm_san.so: tcm_api.cpp with the sanitizers (g++), linked by
    g++ with the device objects of an ordinary build (built here if absent)."""
    os.makedirs(BUILD, exist_ok=True)
    dev = [s for s in SOURCES if s.endswith(".hip")]
    objs = [os.path.join(BUILD, s + ".o") for s in dev]
    missing = [s for s, o in zip(dev, objs) if not os.path.exists(o)]
    with cf.ThreadPoolExecutor(max_workers=max(1, len(missing))) as ex:
        list(ex.map(lambda s: _compile(s, None), missing))
    host = _compile("tcm_api.cpp", None, sanitize=True)
    subprocess.run(["g++", "-shared", *SANITIZE, host, *objs, "-o", SAN_LIB,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly here")
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="build _build/libtcm_san.so (host code with ASan/UBSan) instead")
    a = ap.parse_args(argv)
    if a.clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    if a.sanitize:
        build_sanitized()
    else:
        build(a.asm)
    return 0


if __name__ == "__main__":
    sys.exit(main())
