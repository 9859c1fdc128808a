"""Builds the library's HIP sources as host C++ against the emulator runtime:
tests/emu/_build/libmla_emu.so exports the same C ABI as libmla.so, with every
kernel run on the CPU by the emulator.  Test infrastructure only.

    python -m tests.emu.build_emu
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "head_latent_attention_05_amd", "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmla_emu.so")
CXX = os.environ.get("EMU_CXX", "/opt/rocm/llvm/bin/clang++")

FLAGS = [
    "-std=c++17", "-O2", "-g", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unknown-pragmas", "-Wno-unused-variable", "-Wno-pass-failed",
    "-fno-strict-aliasing",
    # out-of-range indexing of fixed-size arrays (register tiles, LDS arrays) traps
    "-fsanitize=bounds", "-fsanitize-trap=all",
    "-I", os.path.join(HERE, "include"),
]


def _sources(csrc: str = CSRC):
    hips = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    return hips, [os.path.join(HERE, "emu_runtime.cpp")]


def _stamp(csrc: str = CSRC) -> str:
    h = hashlib.sha256()
    hips, cpps = _sources(csrc)
    deps = hips + cpps + sorted(glob.glob(os.path.join(csrc, "*.h")))
    deps += sorted(glob.glob(os.path.join(HERE, "include", "**", "*.h"), recursive=True))
    deps += [os.path.join(ROOT, "include", "mla.h"), os.path.abspath(__file__)]
    for p in deps:
        h.update(p.encode())
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def _compile(args):
    src, is_hip, out_dir = args
    obj = os.path.join(out_dir, os.path.basename(src) + ".emu.o")
    cmd = [CXX, *FLAGS]
    if is_hip:
        cmd += ["-x", "c++", "-include", "emu_gfx950_asm.h"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"emulator build failed for {src}:\n{r.stderr}")
    return obj


def build(force: bool = False, csrc: str = CSRC, out_dir: str = OUT_DIR) -> str:
    """Build the emulated library from the kernel sources in `csrc` (default:
    the library's own) into `out_dir`; rebuilt only when a source changed.
    Concurrent builds (parallel test workers) serialise on a lock file."""
    import fcntl

    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libmla_emu.so")
    with open(os.path.join(out_dir, "lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        stamp = _stamp(csrc)
        stamp_file = os.path.join(out_dir, "stamp")
        if not force and os.path.exists(lib) and os.path.exists(stamp_file):
            with open(stamp_file) as f:
                if f.read() == stamp:
                    return lib
        hips, cpps = _sources(csrc)
        jobs = [(s, True, out_dir) for s in hips] + [(s, False, out_dir) for s in cpps]
        with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            objs = list(ex.map(_compile, jobs))
        tmp = lib + ".tmp"
        r = subprocess.run([CXX, "-shared", "-fPIC", "-o", tmp, *objs], capture_output=True,
                           text=True)
        if r.returncode != 0:
            raise RuntimeError(f"emulator link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        with open(stamp_file, "w") as f:
            f.write(stamp)
    return lib


if __name__ == "__main__":
    print(build(force=True))
