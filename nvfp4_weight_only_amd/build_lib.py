"""Builds libqerl_nvfp4.so (the HIP library behind include/qerl_nvfp4.h) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqerl_nvfp4.so")
SOURCES = ["quantize.hip", "linear.hip", "norm.hip", "misc.hip", "backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed FP32 VALU forms are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


# The library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code (the device code is built as
# usual and never run by the sanitizer test), for the sanitizer test of the C ABI's host logic: validation, plans,
# workspace layouts. The objects leave the sanitizer runtime's symbols to the process, which preloads it. Rebuilt
# only when a source is newer than the library.
SANITIZE_HOST = ["-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_DIR = os.path.join(HERE, "_build_san")


def build_host_sanitized(outdir: str = SAN_DIR) -> str:
    os.makedirs(outdir, exist_ok=True)
    out = os.path.join(outdir, "libqerl_nvfp4_host_san.so")
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "qerl_nvfp4.h")]
    if os.path.exists(out) and os.path.getmtime(out) >= max(os.path.getmtime(d) for d in deps):
        return out

    def compile_one(src):
        obj = os.path.join(outdir, src.replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *FLAGS, *SANITIZE_HOST, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of hipcc's compiler (to preload in the process that loads the build)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = found[0] if found else ""
    return path


if __name__ == "__main__":
    print(build(verbose=True))
