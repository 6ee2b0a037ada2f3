"""Builds liblorabwd.so (HIP, gfx950) in-tree with hipcc.

`python -m layer_backward_pass_amd._build --sanitize` builds a second copy,
_build_san/liblorabwd_san.so, whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (device code as usual); load it through the
LORABWD_LIB environment variable with the sanitizer runtime preloaded
(tests/test_sanitized_abi.py does this for the C-ABI validation tests)."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["rowwise.hip", "gemm.hip", "decode.hip", "attn.hip", "lora.hip", "lmhead.hip",
           "api.hip"]
LIB = os.path.join(HERE, "liblorabwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (v_pk_* fp32 forms are avoided)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# host-only sanitizer flags (each -fsanitize= applies to the host pass only)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_DIR = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "liblorabwd_san.so")


def sanitizer_runtime():
    """The clang AddressSanitizer runtime to preload into an uninstrumented
    Python (None if the toolchain has none)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def _compile(src, out_dir, extra=()):
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose=False):
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def build_sanitized(verbose=False):
    os.makedirs(SAN_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, SAN_DIR, SAN_FLAGS), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *SAN_FLAGS,
           *objs, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    import sys
    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
