"""Host-side AddressSanitizer build of libvla (CPU checks only).

The host runtime (api.cpp: validation, workspace plans, graph caches, fused
plans) is compiled with ASan on the host side only; the device code and the
kernel objects are the normal build's. The result, _build/asan/libvla.so,
is for running the host-side tests (argument validation, workspace sizing)
under ASan on a machine without a GPU: load it through VLA_LIB_PATH with the
ASan runtime preloaded (see asan_env()).
"""

from __future__ import annotations

import os
import subprocess

from . import build as _b

ASAN_DIR = os.path.join(_b.BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libvla.so")
CLANG = os.environ.get("VLA_CLANG", "/opt/rocm/lib/llvm/bin/clang")


def runtime() -> str:
    return subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build_asan() -> str:
    """Compile api.cpp with host-side ASan and link it with the normal kernel
    objects (built first when missing)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = [os.path.join(_b.BUILD, s + ".o") for s in _b.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _b.build(verbose=False)
    api_o = os.path.join(ASAN_DIR, "api.cpp.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [_b.HIPCC] + _b.FLAGS + host_asan + ["-x", "hip", "-c", os.path.join(_b.CSRC, "api.cpp"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan compile failed\n{r.stderr}")
    link = [_b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
            "-shared-libasan", "-o", ASAN_LIB, api_o] + objs
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan link failed\n{r.stderr}")
    return ASAN_LIB


def asan_env() -> dict:
    env = dict(os.environ)
    env["VLA_LIB_PATH"] = ASAN_LIB
    env["LD_PRELOAD"] = runtime()
    # the Python interpreter itself is not instrumented: leaks of the
    # interpreter and the HIP runtime are not ours to report
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    return env


if __name__ == "__main__":
    print(build_asan())
