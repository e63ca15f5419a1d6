"""Build libsnip.so (the HIP kernels and the C ABI) in-tree for gfx950.

Run `python -m sub_byte_mixed_amd.build` or call build(); it always
recompiles. hipcc flags: -ffp-contract=off keeps the fp32 rounding sequence
of the quantizers bit-exact, -fno-gpu-flush-denormals-to-zero keeps fp32
subnormals, and the packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsnip.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.hip", "quantize.hip", "quantize_dual.hip", "quantize_fp4v.hip", "gemm.hip", "gemm_staged.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


REPO = os.path.dirname(HERE)
HELPERS = os.path.join(REPO, "tests", "helpers")
CHECKER_SRC = os.path.join(HELPERS, "hw_convert_check.hip")
CHECKER_BIN = os.path.join(HELPERS, "hw_convert_check")
MFMA_PROBE_SRC = os.path.join(HELPERS, "fp8_mfma_accuracy.hip")
MFMA_PROBE_BIN = os.path.join(HELPERS, "fp8_mfma_accuracy")
CLOCK_PROBE_SRC = os.path.join(HELPERS, "mfma_clock.hip")
CLOCK_PROBE_BIN = os.path.join(HELPERS, "mfma_clock")


def _build_helper(src: str, out: str, verbose: bool, extra=()) -> str:
    cmd = [hipcc_path(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], *extra, "-o", out + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    os.replace(out + ".tmp", out)
    return out


ASAN_SRC = os.path.join(HELPERS, "abi_asan_check.cpp")
ASAN_BIN = os.path.join(HELPERS, "abi_asan_check")


def build_asan_check(verbose: bool = False) -> str:
    """The library's sources and tests/helpers/abi_asan_check.cpp as one
    executable whose host code is built with AddressSanitizer and
    UndefinedBehaviorSanitizer (device code is not instrumented): the
    validation and sizing paths of every entry point, checked on the CPU."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    base = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-O3")] + ["-O1", "-g"]

    def one(src):
        obj = os.path.join(BUILD_DIR, "asan_" + os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc_path(), *base, *san, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        return obj

    from concurrent.futures import ThreadPoolExecutor
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [ASAN_SRC]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, srcs))
    cmd = [hipcc_path(), "--offload-arch=gfx950", *san, "-o", ASAN_BIN + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(ASAN_BIN + ".tmp", ASAN_BIN)
    return ASAN_BIN


def build_checker(verbose: bool = False) -> str:
    """The GPU test and measurement helpers: the exhaustive hardware-convert
    checker, the FP8 matrix-instruction accuracy probe and the shader-clock
    probe."""
    _build_helper(MFMA_PROBE_SRC, MFMA_PROBE_BIN, verbose)
    # accumulators in VGPRs: the AGPR form costs register copies in its loop
    _build_helper(CLOCK_PROBE_SRC, CLOCK_PROBE_BIN, verbose, ("-mllvm", "-amdgpu-mfma-vgpr-form=true"))
    return _build_helper(CHECKER_SRC, CHECKER_BIN, verbose)


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc_path(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-c", "-o", obj, os.path.join(CSRC, src)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if res.returncode != 0:
        errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj


# Kernels that issue MFMAs as inline asm, per source: their device assembly
# is checked for the wait states the compiler does not insert for them
# (asm_hazards.py); a violation fails the build.
ASM_MFMA_KERNELS = {"gemm.hip": ["gemm_nvfp4_w1_kernel", "gemm_mxfp4_w1_kernel", "gemm_mxfp4_w1p_kernel"]}


def _device_asm(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".device.s")
    cmd = [hipcc_path(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-S", "--cuda-device-only", "-o", out,
           os.path.join(CSRC, src)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if res.returncode != 0:
        errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc -S failed on {src}:\n{errs}")
    return out


def check_asm_mfma(asm_path: str, kernels) -> None:
    """Raise if a listed kernel is missing or breaks an asm-MFMA hazard bound."""
    from . import asm_hazards
    text = open(asm_path).read()
    for part in kernels:
        res = asm_hazards.check_asm(text, part)
        if not res or not all(n > 0 for n, _ in res.values()):
            raise RuntimeError(f"{asm_path}: no asm MFMAs found in kernels matching {part!r}")
        for name, (_, bad) in res.items():
            if bad:
                raise RuntimeError(f"{asm_path}: {name}: asm MFMA hazard:\n  " + "\n  ".join(bad[:10]))


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), check the device
    assembly of the asm-MFMA kernels, then link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [("o", s) for s in SOURCES] + [("s", s) for s in ASM_MFMA_KERNELS]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda j: _compile(j[1], verbose) if j[0] == "o" else _device_asm(j[1], verbose), jobs))
    objs = outs[:len(SOURCES)]
    for (kind, src), path in zip(jobs, outs):
        if kind == "s":
            check_asm_mfma(path, ASM_MFMA_KERNELS[src])
    out_tmp = LIB + ".tmp"
    cmd = [hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if os.path.exists(CHECKER_SRC):
        print(build_checker(verbose="-v" in sys.argv))
