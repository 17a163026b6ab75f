"""Build libdocmask_gqa.so (HIP, gfx950) in place with hipcc.

    python -m context_gqa_amd.build

Compiles every csrc/*.hip translation unit in parallel and links the shared
library next to this file.  Always recompiles (no stale-object reuse).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdocmask_gqa.so")
ARCH = os.environ.get("DMGQA_OFFLOAD_ARCH", "gfx950")

# Packed FP32 (v_pk_*_f32) is disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build")
    return path


def _filter(out: str) -> str:
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra=None, out: str = LIB, link_extra=None) -> str:
    """Compile every csrc/*.hip and link the shared library at `out`.
    extra: more compile flags; link_extra: more link flags (the sanitizer
    build of the host code uses both)."""
    cc = hipcc()
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    tmp = tempfile.mkdtemp(prefix="dmgqa_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *COMMON, *DEVICE_FLAGS, *(extra or []), "-c",
                   os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{_filter(r.stderr)}")
            if verbose and _filter(r.stderr).strip():
                print(_filter(r.stderr))
            return obj

        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp_lib = os.path.join(tmp, "libdocmask_gqa.so")
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *(link_extra or []), *objs,
               "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
        shutil.move(tmp_lib, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


# Host-only AddressSanitizer and UndefinedBehaviorSanitizer: each -fsanitize
# flag applies to the host compilation only (-Xarch_host); device code is
# built as usual.  The library then needs the shared ASan runtime
# (-shared-libasan), which the process must preload.
SANITIZE_COMPILE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                    "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan", "-O1"]
SANITIZE_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime of this toolchain."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("shared ASan runtime not found")
    return path


def build_sanitized(out: str) -> str:
    """The library with the host code built under ASan and UBSan."""
    return build(extra=SANITIZE_COMPILE, out=out, link_extra=SANITIZE_LINK)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
