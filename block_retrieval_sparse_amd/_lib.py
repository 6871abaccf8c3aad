"""ctypes binding of libbrs (the HIP C-ABI library declared in include/brs.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  Importing
this module fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

# always the in-tree build next to this file
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbrs.so")

BRS_F32, BRS_BF16 = 0, 1
REP_MEAN, REP_TOPNORM, REP_GIVEN, REP_EMBED, REP_ATTNSCORE = 0, 1, 2, 3, 4
REP_MODES = {"mean": REP_MEAN, "topnorm": REP_TOPNORM, "given": REP_GIVEN, "embed": REP_EMBED,
             "attnscore": REP_ATTNSCORE}
ERRORS = {0: "BRS_OK", -1: "BRS_E_INVAL", -2: "BRS_E_CAPACITY", -3: "BRS_E_UNSUPPORTED",
          -4: "BRS_E_HIP", -5: "BRS_E_EMPTY", -6: "BRS_E_WORKSPACE"}

# every symbol include/brs.h and include/brs_measure.h declare
EXPORTS = ["brs_version", "brs_last_error", "brs_memory_check", "brs_mem_append", "brs_eligible_range",
           "brs_score_blocks", "brs_score_blocks_group", "brs_select_topk", "brs_attention_workspace_bytes",
           "brs_retrieval_attention", "brs_retrieval_step", "brs_window_mass", "brs_reps_from_mass",
           "brs_count_hits", "brs_mem_prune", "brs_profile_next_attention", "brs_measure_read",
           "brs_retrieval_step_static", "brs_static_scratch_bytes", "brs_cache_reset", "brs_cache_fetch",
           "brs_retrieval_attention_cached"]


class brs_memory(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("batch", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
        ("row_stride", c_int32), ("block_size", c_int32), ("reps_per_block", c_int32),
        ("rep_dim", c_int32), ("rep_heads", c_int32), ("rep_mode", c_int32), ("rep_dtype", c_int32),
        ("reserved", c_int32), ("capacity", c_int64), ("length", c_int64),
        ("k", c_void_p), ("v", c_void_p), ("reps", c_void_p),
    ]


class brs_page_cache(ctypes.Structure):
    _fields_ = [
        ("k", c_void_p), ("v", c_void_p), ("page_of_block", c_void_p), ("page_block", c_void_p),
        ("page_rows", c_void_p), ("page_used", c_void_p), ("n_pages", c_int32), ("reserved", c_int32),
    ]


class BrsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_retrieval_sparse_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER(brs_memory)
    sig = {
        "brs_version": (c_int, []),
        "brs_last_error": (ctypes.c_char_p, []),
        "brs_memory_check": (c_int, [P]),
        "brs_mem_append": (c_int, [P, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
        "brs_eligible_range": (c_int, [P, c_int64, c_int64, POINTER(c_int64), POINTER(c_int64)]),
        "brs_score_blocks": (c_int, [P, c_void_p, c_int32, c_int64, c_int64, c_void_p, c_void_p]),
        "brs_score_blocks_group": (c_int, [P, c_void_p, c_int32, c_int64, c_int64, c_void_p, c_void_p]),
        "brs_select_topk": (c_int, [c_void_p, c_int32, c_int32, c_int64, c_int64, c_int64, c_int32,
                                    c_void_p, c_void_p, c_void_p]),
        "brs_attention_workspace_bytes": (c_int, [P, c_int32, c_int32, c_int32, c_int32, c_int64, c_int64,
                                                  POINTER(c_size_t)]),
        "brs_retrieval_attention": (c_int, [P, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                            c_int64, c_int64, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                            c_void_p]),
        "brs_retrieval_step": (c_int, [P, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_int64, c_int64,
                                       c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                       c_void_p]),
        "brs_window_mass": (c_int, [P, c_void_p, c_int32, c_int32, c_void_p, c_int64, c_float, c_void_p,
                                    c_void_p]),
        "brs_reps_from_mass": (c_int, [P, c_void_p, c_int64, c_int64, c_void_p]),
        "brs_count_hits": (c_int, [P, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
        "brs_mem_prune": (c_int, [P, c_void_p, P, c_void_p, c_void_p, c_void_p]),
        "brs_profile_next_attention": (c_int, [c_void_p, c_void_p]),
        "brs_measure_read": (c_int, [c_void_p, c_int64, c_void_p, c_int64, ctypes.c_uint32, c_void_p, c_void_p]),
        "brs_retrieval_step_static": (c_int, [P, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_int64,
                                              c_int64, c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p]),
        "brs_static_scratch_bytes": (c_size_t, []),
        "brs_cache_reset": (c_int, [P, POINTER(brs_page_cache), c_void_p]),
        "brs_cache_fetch": (c_int, [P, POINTER(brs_page_cache), c_void_p, c_int32, c_int32, c_int64, c_int64, c_int32,
                                    c_void_p, c_void_p]),
        "brs_retrieval_attention_cached": (c_int, [P, POINTER(brs_page_cache), c_void_p, c_int32, c_int32, c_void_p,
                                                   c_int32, c_int32, c_int64, c_int64, c_float, c_void_p, c_void_p,
                                                   c_void_p, c_size_t, c_void_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def check(rc: int) -> None:
    if rc != 0:
        raise BrsError(rc, lib.brs_last_error().decode())
