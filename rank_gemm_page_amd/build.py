"""Compile the HIP library (host runtime + gfx950 kernels) into libslora.so, in tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libslora.so")
SOURCES = ["slora_host.cpp", "slora_kernels.hip", "slora_forward.hip", "slora_probe.hip", "slora_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are switched off for the device code: plain float code
# is compiled to scalar-per-lane fp32 instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libslora.so next to this file."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SANITIZED_LIB_PATH = os.path.join(PKG_DIR, "libslora_sanitized.so")


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime, to preload into a process that
    loads the sanitized library."""
    clangxx = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    out = subprocess.run([clangxx, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """libslora with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (every undefined-behaviour report is fatal);
    the device code is built as usual.  For CPU tests of the host runtime
    (allocator, segment builder, tile lists, argument checks): load it with
    SLORA_LIB pointing at it and asan_runtime() preloaded."""
    tmp = SANITIZED_LIB_PATH + ".tmp"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libasan", "-g"]
    cmd = [HIPCC, *FLAGS, *san, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized) failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, SANITIZED_LIB_PATH)
    return SANITIZED_LIB_PATH


def device_assembly(workdir: str, source: str = "slora_kernels.hip") -> str:
    """Compile one HIP source for gfx950 keeping the assembly; return its path."""
    src = os.path.join(CSRC, source)
    stem = os.path.splitext(source)[0]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, "--save-temps", "-o", os.path.join(workdir, stem + ".o"), src]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=workdir)
    if res.returncode != 0:
        raise RuntimeError(res.stderr)
    return os.path.join(workdir, f"{stem}-hip-amdgcn-amd-amdhsa-gfx950.s")


def masked_mfma_lines(asm_path: str):
    """Lines of v_mfma instructions that may run under a partial EXEC mask.

    A matrix instruction executes for the whole wavefront regardless of EXEC,
    so one placed after an exec-narrowing instruction, with no s_cbranch_execz,
    label or exec restore in between, would accumulate operands of lanes that
    were meant to be switched off.
    """
    bad, masked = [], False
    with open(asm_path) as f:
        for no, line in enumerate(f, 1):
            t = line.strip()
            parts = t.split()
            op = parts[0] if parts else ""
            dst = parts[1].rstrip(",") if len(parts) > 1 else ""
            if op in ("s_and_saveexec_b64", "s_andn2_saveexec_b64", "s_or_saveexec_b64") or (
                    op.startswith("s_") and dst == "exec" and op != "s_or_b64"
                    and not op.startswith("s_mov")):
                masked = True
            if (op.startswith("s_cbranch_execz") or (op == "s_or_b64" and dst == "exec")
                    or t.endswith(":") or op == "s_branch"
                    or (op.startswith("s_mov") and dst == "exec")):
                masked = False
            if op.startswith("v_mfma") and masked:
                bad.append(no)
    return bad


if __name__ == "__main__":
    print(build(verbose=True))
