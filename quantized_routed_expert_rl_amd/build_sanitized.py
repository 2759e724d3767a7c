"""Build a copy of librlmoe whose host code (the C ABI's argument checks, the
expert cache, the native driver) carries AddressSanitizer and
UndefinedBehaviorSanitizer; device code is compiled as usual.  For tests on
the CPU only: the Python process must preload the ASan runtime
(``asan_runtime()``) and point RLMOE_LIB at the built library.

    python -m quantized_routed_expert_rl_amd.build_sanitized
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from . import build as B

OUT_DIR = os.path.join(B.BUILD, "sanitized")
OUT = os.path.join(OUT_DIR, "librlmoe_sanitized.so")
# each sanitizer flag is scoped to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str | None:
    """The clang ASan runtime that hipcc's host compiler links against, or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src)[:-4] + ".o")
    flags = [f if f != "-O3" else "-O1" for f in B.FLAGS] + ["-g"] + HOST_SAN
    r = subprocess.run([B.HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = B.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = [B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan",
           "-o", OUT, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
