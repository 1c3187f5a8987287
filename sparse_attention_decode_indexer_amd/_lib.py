"""ctypes loader for libnsa.so and the C signatures of include/nsa.h."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# NSA_LIB_PATH selects another build of the same library (the host-sanitizer
# build of the CPU tests); the default is the in-tree libnsa.so
LIB_PATH = os.environ.get("NSA_LIB_PATH") or os.path.join(_PKG, "libnsa.so")

c_int, c_i64, c_f32, c_size = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
P = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/nsa.h
SIGNATURES = {
    "nsa_last_error": (ctypes.c_char_p, []),
    "nsa_version": (c_int, []),
    "nsa_check_device_errors": (c_int, [P]),
    "nsa_build_metadata": (c_int, [
        c_int, c_int, c_int, c_int, c_int, P, P, P, c_i64, c_i64, P, c_int, c_int,
        P, P, P, P, P, P, P, P, c_i64, P, P, c_i64, P]),
    "nsa_indexer_logits": (c_int, [
        P, c_int, P, P, c_int, c_i64, P, c_i64, c_i64, P, P, c_int, c_int, c_int,
        c_int, c_int, P, c_i64, P]),
    "nsa_indexer_logits_hist": (c_int, [
        P, c_int, P, P, c_int, c_i64, P, c_i64, c_i64, P, P, c_int, c_int, c_int,
        c_int, c_int, P, c_i64, P, c_int, P]),
    "nsa_topk_workspace_size": (c_int, [c_int, c_int, c_int, ctypes.POINTER(c_size)]),
    "nsa_topk_hist_workspace_size": (c_int, [c_int, c_int, c_int,
                                             ctypes.POINTER(c_size)]),
    "nsa_topk_transform_hist": (c_int, [
        P, c_i64, P, c_int, c_int, c_int, P, c_i64, c_i64, P, c_int, P, P, c_i64, P,
        c_size, P]),
    "nsa_topk_transform": (c_int, [
        P, c_i64, P, c_int, c_int, c_int, P, c_i64, c_i64, P, c_int, P, c_i64, P,
        c_size, P]),
    "nsa_page_table_transform": (c_int, [
        P, c_i64, c_int, c_int, P, c_i64, c_i64, P, c_i64, c_i64, c_i64, c_int, P, P,
        c_i64, P]),
    "nsa_sparse_mla_workspace_size": (c_int, [c_int, c_int, c_int, c_int,
                                              ctypes.POINTER(c_size)]),
    "nsa_sparse_mla_decode": (c_int, [
        P, c_i64, c_i64, P, c_int, c_i64, P, c_i64, P, c_int, c_int, c_int,
        c_int, c_int, c_f32, P, P, P, c_size, P]),
    "nsa_sparse_mla_extend": (c_int, [
        P, c_i64, c_i64, P, c_int, c_i64, P, c_i64, P, c_int, c_int, c_int,
        c_int, c_int, c_f32, P, P, P, c_size, P]),
    "nsa_sparse_mla_decode_noalloc": (c_int, [
        P, c_i64, c_i64, P, c_int, c_i64, P, c_i64, P, c_int, c_int, c_int,
        c_int, c_int, c_f32, P, P, P]),
    "nsa_quantize_k_cache": (c_int, [P, c_i64, c_i64, P, P]),
    "nsa_set_mla_kv_buffer": (c_int, [P, c_i64, P, c_i64, P, c_int, P, c_int,
                                      c_i64, P]),
    "nsa_ragged_extend_metadata": (c_int, [P, P, c_int, P, P, c_int, P, c_i64,
                                           c_int, P, P, P, P, c_i64, P]),
    "nsa_ragged_index_transform": (c_int, [P, c_i64, c_int, c_int, P, P, c_i64, P]),
    "nsa_dequantize_k_cache_paged": (c_int, [P, c_i64, P, c_i64, P, c_i64, P]),
    "nsa_valid_kv_indices": (c_int, [P, c_i64, c_int, c_int, P, P, c_i64, P]),
}

_lib = None


class NsaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load():
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python -m sparse_attention_decode_indexer_amd.build` "
            "(or __graft_entry__.build()). There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def call(name, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise NsaError(name, st, lib.nsa_last_error().decode())
    return st
