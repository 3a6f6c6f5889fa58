"""ctypes declarations of libse.so (the C ABI in include/se.h). Argument marshalling only."""
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libse.so")

# status codes (include/se.h)
(SE_OK, SE_ERR_NULL, SE_ERR_SHAPE, SE_ERR_DTYPE, SE_ERR_PARAM, SE_ERR_WORKSPACE, SE_ERR_UNSUPPORTED, SE_ERR_HIP,
 SE_ERR_SCRATCH_LIMIT) = range(9)
SE_NOALLOC_SCRATCH_BYTES = 16 << 20
SE_DEV_INDEX = 1 << 8
SE_DEV_CAPACITY = 1 << 9
SE_DTYPE_F32, SE_DTYPE_BF16 = 0, 1
SE_SCORE_CAUSAL, SE_SCORE_BIDIR = 0, 1
SE_TOPK_LARGEST, SE_TOPK_SMALLEST = 0, 1
SE_UNIT_SLOT, SE_UNIT_PAGE = 0, 1
SE_COMPACT_GATHER, SE_COMPACT_EVICT_SLOTS = 0, 1
SE_PAGES_BUILD, SE_PAGES_SCORE = 0, 1
SE_REFRESH_LAST_PAGE, SE_REFRESH_FROM_PAGE = 0, 1

P = C.c_void_p
I32 = C.c_int32


class se_cache_t(C.Structure):
    _fields_ = [
        ("k_pool", P), ("v_pool", P), ("block_table", P), ("pos_map", P), ("ctx_len", P), ("n_slots", P),
        ("free_blocks", P), ("free_top", P), ("slot_stack", P), ("slot_top", P), ("page_meta", P),
        ("cum_score", P),
        ("B", I32), ("n_kv", I32), ("n_q", I32), ("d", I32), ("page", I32), ("num_blocks", I32),
        ("max_blocks", I32), ("slot_cap", I32), ("dtype", I32),
    ]


class se_window_params_t(C.Structure):
    _fields_ = [("scale", C.c_float), ("mode", I32), ("n_query", I32), ("window", I32), ("protect", I32),
                ("score_stride", I32), ("accumulate", I32)]


class se_topk_params_t(C.Structure):
    _fields_ = [("mode", I32), ("unit", I32), ("k", I32), ("window", I32), ("protect", I32), ("forced_ends", I32),
                ("budget", I32), ("recent", I32), ("score_stride", I32), ("out_stride", I32), ("range_lo", I32),
                ("range_hi", I32), ("emit_dropped", I32), ("block_refs", C.c_void_p)]


class se_t2c_params_t(C.Structure):
    _fields_ = [("max_gap", I32), ("budget", I32), ("window", I32), ("protect", I32), ("score_stride", I32),
                ("in_stride", I32), ("out_stride", I32)]


class se_compact_params_t(C.Structure):
    _fields_ = [("mode", I32), ("window", I32), ("idx_stride", I32)]


class se_decode_params_t(C.Structure):
    _fields_ = [("scale", C.c_float), ("sel_stride", I32), ("max_sel", I32), ("max_slots", I32),
                ("accumulate", I32)]


class se_h2o_params_t(C.Structure):
    _fields_ = [("scale", C.c_float), ("budget", I32), ("recent", I32)]


EXPORTS = {
    "se_window_score_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), C.POINTER(se_window_params_t)]),
    "se_window_score": (I32, [C.POINTER(se_cache_t), P, P, C.POINTER(se_window_params_t), P, P, P, C.c_size_t, P]),
    "se_topk_select_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), C.POINTER(se_topk_params_t)]),
    "se_topk_select": (I32, [C.POINTER(se_cache_t), P, C.POINTER(se_topk_params_t), P, P, P, P, C.c_size_t, P]),
    "se_token2chunk": (I32, [C.POINTER(se_cache_t), P, P, P, C.POINTER(se_t2c_params_t), P, P, P, P, C.c_size_t,
                             P]),
    "se_compact_evict_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), C.POINTER(se_compact_params_t)]),
    "se_compact_evict": (I32, [C.POINTER(se_cache_t), P, P, C.POINTER(se_compact_params_t), P, P, C.c_size_t, P]),
    "se_cache_append_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t)]),
    "se_cache_append": (I32, [C.POINTER(se_cache_t), P, P, P, P, P, C.c_size_t, P]),
    "se_cache_append_chunk_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), I32]),
    "se_cache_append_chunk": (I32, [C.POINTER(se_cache_t), P, P, P, I32, P, P, P, C.c_size_t, P]),
    "se_page_bounds": (I32, [C.POINTER(se_cache_t), I32, P, P, I32, P, P, C.c_size_t, P]),
    "se_page_bounds_refresh": (I32, [C.POINTER(se_cache_t), I32, P, I32, P, P, C.c_size_t, P]),
    "se_sparse_decode_attn_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), C.POINTER(se_decode_params_t),
                                                          I32]),
    "se_sparse_decode_attn": (I32, [C.POINTER(se_cache_t), P, P, P, C.POINTER(se_decode_params_t), P, P, P,
                                    C.c_size_t, P]),
    "se_sparse_decode_attn_noalloc": (I32, [C.POINTER(se_cache_t), P, P, P, C.POINTER(se_decode_params_t), P, P,
                                            P]),
    "se_h2o_decode_evict_workspace_size": (C.c_size_t, [C.POINTER(se_cache_t), C.POINTER(se_h2o_params_t)]),
    "se_h2o_decode_evict": (I32, [C.POINTER(se_cache_t), P, C.POINTER(se_h2o_params_t), P, P, P, P, P, C.c_size_t,
                                  P]),
    "se_status_read": (I32, [P, C.POINTER(I32), I32, P]),
    "se_error_string": (C.c_char_p, [I32]),
    "se_version": (C.c_char_p, []),
}

_lib = None


def load():
    """Load libse.so (built in place by ``python -m sparse_decode_attention_se_amd.build``). Raises if missing:
    there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m sparse_decode_attention_se_amd.build")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
