"""Build libvw4.so (HIP, gfx950) in-tree.

Every .hip file under csrc/ is compiled with hipcc for gfx950 into an object
(in parallel), then linked into verify_step_w4_amd/libvw4.so.  Packed-FP32
instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvw4.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = os.environ.get("VW4_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


# Host-side AddressSanitizer / UndefinedBehaviorSanitizer for a CPU check of
# the ABI's host code (argument validation, host quantisers, plans): each
# -fsanitize= applies to the host pass only; the device code is built as usual.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile every csrc/*.hip and link `out` (default libvw4.so).  With
    sanitize, the host code carries ASan + UBSan (objects in a build folder
    of their own); load such a library only in a process that preloads the
    compiler's ASan runtime first."""
    build_dir = BUILD_DIR + ("_san" if sanitize else "")
    extra = SANITIZE_HOST if sanitize else ()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(verbose=True)
