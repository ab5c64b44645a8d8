"""ctypes declarations for libmla.so (the C ABI in include/mla.h).

Loading fails loudly: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_ABSORBED, MLA_MATERIALIZED = 0, 1
STATUS = {0: "MLA_OK", -1: "MLA_E_NULL", -2: "MLA_E_SHAPE", -3: "MLA_E_UNSUPPORTED",
          -4: "MLA_E_WORKSPACE", -5: "MLA_E_HIP"}

# Every symbol include/mla.h declares.
EXPORTS = ("mla_status_string", "mla_version", "mla_select_path", "mla_draft_cap", "mla_fold_query",
           "mla_absorbed_workspace_size", "mla_absorbed_attention", "mla_absorbed_attention_noalloc",
           "mla_absorbed_splits",
           "mla_absorbed_merge", "mla_materialize_kv",
           "mla_materialized_workspace_size", "mla_materialized_attention", "mla_quantize_latent_fp8",
           "mla_absorbed_attention_fp8", "mla_absorbed_splits_fp8", "mla_query_fp8_bytes", "mla_fold_query_fp8",
           "mla_absorbed_attention_fp8q", "mla_absorbed_splits_fp8q", "mla_absorbed_sparse_workspace_size",
           "mla_absorbed_attention_sparse", "mla_absorbed_attention_sparse_fp8", "mla_indexer_pool_init", "mla_indexer_pool_plan",
           "mla_indexer_pool_step", "mla_indexer_update_list", "mla_indexer_pool_step_fixed", "mla_indexer_pool_trim", "mla_indexer_scores", "mla_indexer_pool_step_scores",
           "mla_indexer_selection_offsets", "mla_indexer_select")


class Geom(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("n", ctypes.c_int32), ("v", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("heads", ctypes.c_int32)]

    def __repr__(self):
        return f"Geom(r={self.r}, n={self.n}, v={self.v}, rope={self.rope}, heads={self.heads})"


class Pool(ctypes.Structure):
    """mla_pool: host-side state of the indexer's pooled keys."""
    _fields_ = [("pooled", ctypes.c_void_p), ("capacity", ctypes.c_int32), ("batch_max", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("d", ctypes.c_int32), ("valid", ctypes.c_int32),
                ("lengths", ctypes.POINTER(ctypes.c_int32))]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None

VP = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
GP = ctypes.POINTER(Geom)
I32P = ctypes.POINTER(ctypes.c_int32)
I64P = ctypes.POINTER(ctypes.c_int64)
SZP = ctypes.POINTER(ctypes.c_size_t)


def load() -> ctypes.CDLL:
    """Load libmla.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mla_speculative_decode_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_version.restype = ctypes.c_int
    lib.mla_version.argtypes = []
    lib.mla_select_path.restype = ctypes.c_int
    lib.mla_select_path.argtypes = [GP, I64, I64, I32P, I64P]
    lib.mla_draft_cap.restype = ctypes.c_int
    lib.mla_draft_cap.argtypes = [ctypes.POINTER(ctypes.c_double), I32, ctypes.c_double, ctypes.c_double, I32P,
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.mla_fold_query.restype = ctypes.c_int
    lib.mla_fold_query.argtypes = [GP, ctypes.c_int, I64, VP, VP, VP, VP]
    lib.mla_absorbed_workspace_size.restype = ctypes.c_int
    lib.mla_absorbed_workspace_size.argtypes = [GP, ctypes.c_int, I32, I32, VP, SZP]
    lib.mla_absorbed_attention.restype = ctypes.c_int
    lib.mla_absorbed_attention.argtypes = [GP, ctypes.c_int, I32, I32, VP, VP, VP, VP, VP, VP, VP,
                                           ctypes.c_float, VP, VP, ctypes.c_size_t, VP]
    lib.mla_absorbed_attention_noalloc.restype = ctypes.c_int
    lib.mla_absorbed_attention_noalloc.argtypes = [GP, ctypes.c_int, I32, I32, VP, VP, VP, VP, VP, VP, VP,
                                                   ctypes.c_float, VP, VP]
    lib.mla_absorbed_splits.restype = ctypes.c_int
    lib.mla_absorbed_splits.argtypes = [GP, ctypes.c_int, I32, I32, VP, VP, VP, VP, VP, VP, ctypes.c_float,
                                        VP, ctypes.c_size_t, VP]
    lib.mla_absorbed_merge.restype = ctypes.c_int
    lib.mla_absorbed_merge.argtypes = [GP, ctypes.c_int, I32, I32, VP, VP, VP, VP, VP, ctypes.c_size_t, VP]
    lib.mla_materialize_kv.restype = ctypes.c_int
    lib.mla_materialize_kv.argtypes = [GP, ctypes.c_int, I64, VP, VP, VP, VP, VP, VP, VP]
    lib.mla_materialized_workspace_size.restype = ctypes.c_int
    lib.mla_materialized_workspace_size.argtypes = [GP, ctypes.c_int, I32, I32, VP, SZP]
    lib.mla_materialized_attention.restype = ctypes.c_int
    lib.mla_materialized_attention.argtypes = [GP, ctypes.c_int, I32, I32, VP, VP, VP, VP, VP, VP,
                                               ctypes.c_float, VP, VP, ctypes.c_size_t, VP]
    lib.mla_quantize_latent_fp8.restype = ctypes.c_int
    lib.mla_quantize_latent_fp8.argtypes = [GP, I64, VP, VP, VP, VP, VP]
    lib.mla_absorbed_attention_fp8.restype = ctypes.c_int
    lib.mla_absorbed_attention_fp8.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP,
                                               ctypes.c_size_t, VP]
    lib.mla_absorbed_splits_fp8.restype = ctypes.c_int
    lib.mla_absorbed_splits_fp8.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP,
                                            ctypes.c_size_t, VP]
    lib.mla_query_fp8_bytes.restype = ctypes.c_int
    lib.mla_query_fp8_bytes.argtypes = [GP, I32, I32, SZP]
    lib.mla_fold_query_fp8.restype = ctypes.c_int
    lib.mla_fold_query_fp8.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP]
    lib.mla_absorbed_attention_fp8q.restype = ctypes.c_int
    lib.mla_absorbed_attention_fp8q.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP,
                                                ctypes.c_size_t, VP]
    lib.mla_absorbed_splits_fp8q.restype = ctypes.c_int
    lib.mla_absorbed_splits_fp8q.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, ctypes.c_float, VP,
                                             ctypes.c_size_t, VP]
    lib.mla_absorbed_sparse_workspace_size.restype = ctypes.c_int
    lib.mla_absorbed_sparse_workspace_size.argtypes = [GP, I32, I32, VP, VP, SZP]
    lib.mla_absorbed_attention_sparse.restype = ctypes.c_int
    lib.mla_absorbed_attention_sparse.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP,
                                                  ctypes.c_float, VP, VP, ctypes.c_size_t, VP]
    lib.mla_absorbed_attention_sparse_fp8.restype = ctypes.c_int
    lib.mla_absorbed_attention_sparse_fp8.argtypes = [GP, I32, I32, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP,
                                                      ctypes.c_float, VP, VP, ctypes.c_size_t, VP]
    PP = ctypes.POINTER(Pool)
    for name, args in (("mla_indexer_pool_init", [PP, VP, I32, I32, VP]),
                       ("mla_indexer_pool_plan", [PP, I32, I32, VP, I32, I32, I32P]),
                       ("mla_indexer_pool_step", [PP, I32, I32, VP, I64, VP, VP, I32, I32, I32P, VP]),
                       ("mla_indexer_update_list", [I32, I32, I32, I32, I32, VP, I32P]),
                       ("mla_indexer_pool_step_fixed", [PP, I32, I32, VP, I64, VP, VP, I32, I32, I32, I32P, I32P, VP]),
                       ("mla_indexer_pool_trim", [PP, I32, VP]),
                       ("mla_indexer_scores", [PP, I32, VP, VP, VP, VP, VP]),
                       ("mla_indexer_pool_step_scores", [PP, I32, I32, VP, I64, VP, VP, I32, I32, VP, VP, I32P, VP]),
                       ("mla_indexer_selection_offsets", [I32, VP, I32, VP]),
                       ("mla_indexer_select", [I32, VP, I32, VP, VP, I32, VP, VP, VP])):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise MlaError(fn, status, load().mla_status_string(status).decode())
