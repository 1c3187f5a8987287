"""Builds libnsa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m sparse_attention_decode_indexer_amd.build`` (or call
``build_library()``). Every call recompiles.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libnsa.so")

SOURCES = ["status.cpp", "metadata.hip", "transform.hip", "topk.hip",
           "indexer.hip", "sparse_mla.hip", "sparse_mla_h128.hip", "quant.hip",
           "ragged.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE fp32 division for the fp8 cache encoder (x / scale)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]

# Per-source additions. The indexer consumes every MFMA result in VALU code
# at once: MFMAs that write VGPRs save one v_accvgpr_read per output value
# (the attention kernel keeps its accumulators in AGPRs on purpose, so the
# option is not global).
SOURCE_FLAGS = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the 128-head attention kernel keeps its score accumulators in VGPRs and
    # gives all 256 AGPRs to O (those MFMAs are written in their AGPR form)
    "sparse_mla_h128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                            text=True)


def _finish(proc, what, verbose):
    text, _ = proc.communicate()
    out = "\n".join(line for line in text.splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer: every option is
# scoped to the host compilation with -Xarch_host, so the gfx950 code objects
# are built as usual (GPU sanitizers are not used). For the CPU tests of the
# C ABI's argument checks (tests/test_host_sanitizers.py).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build_library(verbose=False, extra_flags=(), lib_path=None, objdir=None,
                  link_flags=()):
    """Compiles every source to an object (in parallel), then links them.
    lib_path / objdir default to the in-tree libnsa.so and _build/."""
    lib_path = lib_path or LIB_PATH
    objdir = objdir or os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-I", INCLUDE,
               "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        objs.append(obj)
        procs.append((_run(cmd, verbose), src))
    for proc, src in procs:
        _finish(proc, src, verbose)
    tmp = lib_path + ".tmp"
    _finish(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_flags, *objs,
                  "-o", tmp], verbose), "link", verbose)
    os.replace(tmp, lib_path)
    return lib_path


def build_host_sanitized(lib_path, objdir, verbose=False):
    """The same library with host ASan + UBSan (see HOST_SANITIZE)."""
    return build_library(verbose, extra_flags=HOST_SANITIZE, lib_path=lib_path,
                         objdir=objdir, link_flags=HOST_SANITIZE)


if __name__ == "__main__":
    build_library(verbose=True, extra_flags=sys.argv[1:])
    print(LIB_PATH)
