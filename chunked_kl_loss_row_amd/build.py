"""Build libkdchunk.so (HIP, gfx950) in-tree with hipcc.

    python -m chunked_kl_loss_row_amd.build [--verbose]

Compiles every ``csrc/*.hip`` translation unit for gfx950 only and links them
into ``chunked_kl_loss_row_amd/libkdchunk.so`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkdchunk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off: hipcc must not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the argument
# checks, workspace layout and chunk scheduler; device code is built as usual).
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
SANITIZE_LINK = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -shared-libsan".split()


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime a host process preloads to
    load the sanitized library (empty if the toolchain has none)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int = 4, sanitize: bool = False, dest: str = LIB) -> str:
    """Compile and link the library; return its path.  Raises on failure.
    sanitize: host code with AddressSanitizer + UndefinedBehaviorSanitizer
    (-O1 -g), written to `dest` (a process loading it preloads
    sanitizer_runtime())."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    srcs = sources()
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *SANITIZE_FLAGS] if sanitize else FLAGS
    with tempfile.TemporaryDirectory(prefix="kdchunk_build_") as tmp:
        procs, objs = [], []
        for src in srcs:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *flags, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        tmp_lib = os.path.join(tmp, "libkdchunk.so")
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *(SANITIZE_LINK if sanitize else []), *objs,
               "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if out.returncode != 0:
            raise RuntimeError("link failed:\n" + out.stdout)
        shutil.copyfile(tmp_lib, dest + ".tmp")
        os.replace(dest + ".tmp", dest)
    return dest


def _wait(item, verbose):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    # the host pass does not know the packed-fp32 target feature: harmless
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
