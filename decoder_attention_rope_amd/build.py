"""Compile the gfx950 attention library (libgqa.so) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, in parallel, then
linked into decoder_attention_rope_amd/libgqa.so next to this file.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgqa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gqa_api.cpp", "rope.hip", "decode.hip", "decode_mfma.hip", "prefill.hip", "prefill_bwd.hip", "qkv.hip",
           "check.hip", "diag.hip"]

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # Packed-f32 VALU forms stay off: plain f32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-lambda-capture",
]


# Per-source flags. The backward's dK/dV kernel keeps its accumulators in
# plain VGPRs (it fits in 256); the compiler's default accumulator-register
# form made it copy accumulators between register files every step.
SOURCE_FLAGS = {
    "prefill_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


# Host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for the
# host-sanitizer test build; device code is built as usual. Each flag sits
# behind -Xarch_host, so it reaches the host compilation only.
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all",
                       "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src, verbose, build_dir=None, extra=()):
    obj = os.path.join(build_dir or BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-f32 feature; that note is noise.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose=False, jobs=None, out=None, host_sanitize=False):
    """Build the library to `out` (default: the in-tree libgqa.so). With
    host_sanitize the host code is instrumented (objects in their own
    directory next to `out`; the process that loads it preloads clang's
    AddressSanitizer runtime)."""
    lib = out or LIB
    build_dir = BUILD_DIR if out is None else os.path.join(os.path.dirname(out), "_build_san")
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    extra = HOST_SANITIZE_FLAGS if host_sanitize else []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
