"""Compile the HIP sources into ``libattn_decode.so`` (gfx950), in-tree.

Run as ``python -m decode_attention_kv_attn_amd.build``.  Objects go to
``_build/`` at the repository root; the shared library lands next to this
file, where the binding loads it.

``build_host_sanitized()`` makes a second library for the CPU tests: the
translation units whose host code checks arguments and plans launches
(api, mla, append) are compiled with AddressSanitizer and
UndefinedBehaviorSanitizer on their host side only (device code is compiled
as usual), and linked with the ordinary kernel objects.  It is loaded with
the sanitizer runtime preloaded (``host_sanitizer_env``).
"""

import os
import shlex
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn_decode.so")

SOURCES = ["api.hip", "gqa_valu.hip", "gqa_valu_global.hip", "gqa_valu_paged.hip",
           "gqa_mfma.hip", "combine.hip", "mla.hip", "mla_mfma.hip", "mla_pair.hip", "append.hip",
           "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # plain float code only: keep the compiler from forming packed-FP32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-side sanitizers (each -fsanitize= right after -Xarch_host: host code only)
SAN_FLAGS = shlex.split("-Xarch_host -fsanitize=address,undefined "
                        "-Xarch_host -fno-omit-frame-pointer -g")
SAN_SOURCES = ["api.hip", "mla.hip", "append.hip"]
SAN_DIR = os.path.join(OBJ, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "libattn_decode_hostsan.so")


def _compile(src, out_dir=OBJ, extra=()):
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def _stale(obj, src):
    return (not os.path.exists(obj) or
            os.path.getmtime(obj) < max(os.path.getmtime(os.path.join(CSRC, f))
                                        for f in os.listdir(CSRC)))


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime (shared) of this toolchain,
    or None."""
    base = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))),
                        "llvm", "lib", "clang")
    if not os.path.isdir(base):
        base = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def host_sanitizer_env(env=None):
    """Environment that loads the host-sanitized library with its runtime."""
    env = dict(os.environ if env is None else env)
    env["LD_PRELOAD"] = sanitizer_runtime()
    env["ATTN_DECODE_LIBRARY"] = SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def build_host_sanitized(verbose=False):
    """The host-sanitized library (see the module docstring)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    os.makedirs(OBJ, exist_ok=True)
    plain = [s for s in SOURCES if s not in SAN_SOURCES]
    todo = [s for s in plain if _stale(os.path.join(OBJ, os.path.splitext(s)[0] + ".o"), s)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(_compile, todo))
        san = list(ex.map(lambda s: _compile(s, SAN_DIR, SAN_FLAGS), SAN_SOURCES))
    objs = san + [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in plain]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS,
           "-shared-libsan", *objs, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
