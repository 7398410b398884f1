"""Compile the HIP sources under csrc/ into libmoba.so (gfx950) next to this file,
and the benchmark's MFMA-rate probe (bench_support/probe.hip) into
bench_support/libmoba_probe.so."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoba.so")
BENCH_SUPPORT = os.path.join(ROOT, "bench_support")
PROBE_SRC = os.path.join(BENCH_SUPPORT, "probe.hip")  # the benchmark's MFMA-rate probe
PROBE_LIB = os.path.join(BENCH_SUPPORT, "libmoba_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "prep.hip", "gate.hip", "dispatch.hip", "attn.hip", "decode.hip", "bwd.hip",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + os.path.join(ROOT, "include"),
    # packed fp32 instructions stay off: the compiler must not emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False) -> str:
    """Always recompiles every source (the result is the build check)."""
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
        out = _run([HIPCC] + FLAGS + ["-c", path, "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES) + 1, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES + [PROBE_SRC]))
    for lib, parts in ((LIB, objs[:-1]), (PROBE_LIB, objs[-1:])):
        tmp = lib + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + parts)
        os.replace(tmp, lib)
    return LIB


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (each flag
# after -Xarch_host: the device code is built as usual, without them).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(out_dir: str) -> str:
    """libmoba.so with sanitized host code, into out_dir (load it with the
    clang ASan runtime preloaded)."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE_FLAGS

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        _run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, "libmoba.so")
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + SANITIZE_FLAGS[:4] +
         ["-Xarch_host", "-shared-libsan", "-o", lib] + objs)
    return lib


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized builds need preloaded."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang ASan runtime not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    print(build(verbose=True))
