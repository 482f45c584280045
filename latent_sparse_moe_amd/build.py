"""Build the HIP library ``_lib/libmoe_latent.so`` for gfx950 with hipcc.

Each ``csrc/*.hip`` compiles to an object in parallel, then one link step
produces the shared library. Packed fp32 instructions are disabled for all
device code (``-target-feature -packed-fp32-ops``).

``--sanitize`` builds a second copy, ``_build/san/libmoe_latent.so``, whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer checks (the
device code is built exactly as in the product library). It is for the CPU:
``tests/host_sanitizers.sh`` loads it in place of the product library and runs
the host-side ABI tests under the sanitizer runtime."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libmoe_latent.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_latent.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-result",
]
# host pass only: every -fsanitize= sits right after its -Xarch_host
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g",
]


def _compile(src: str, obj_dir: str = OBJ_DIR, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature name: drop that note
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile and link the library; returns its path. With ``sanitize`` the
    sanitizer copy is built instead (its sanitizer runtime is not linked in:
    the process that loads it preloads the runtime)."""
    out = SAN_LIB if sanitize else LIB
    obj_dir = os.path.join(ROOT, "_build", "obj_san") if sanitize else OBJ_DIR
    extra = SAN_FLAGS if sanitize else ()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
