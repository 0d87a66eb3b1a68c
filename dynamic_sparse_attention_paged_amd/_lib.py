"""ctypes view of libdsa.so (the C ABI declared in include/dsa.h)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK = 0
STATUS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_UNSUPPORTED",
          -4: "DSA_ERR_ALIGN", -5: "DSA_ERR_WORKSPACE", -6: "DSA_ERR_HIP"}
OP_ATTN_DECODE = 1
OP_DECODE_FUSED = 2
OP_INDEX_TOPK = 3
OP_PREFILL_FUSED = 4
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # DSA_NOALLOC_SCRATCH_BYTES

EXPORTS = ["dsa_index_score", "dsa_topk_blocks", "dsa_sparse_attn_decode",
           "dsa_sparse_attn_decode_topk",
           "dsa_sparse_attn_prefill", "dsa_sparse_decode_fused", "dsa_sparse_decode_fused_noalloc",
           "dsa_sparse_prefill_fused",
           "dsa_index_topk",
           "dsa_workspace_size", "dsa_check_inputs", "dsa_kv_write", "dsa_index_key_write",
           "dsa_mx_quantize", "dsa_mxfp4_to_fp8", "dsa_moe_workspace_size", "dsa_moe_grouped_gemm",
           "dsa_status_str", "dsa_last_error", "dsa_abi_version"]
# include/dsa_support.h: measurement support (ceilings, cache flush, FP8 MFMA probe)
SUPPORT_EXPORTS = ["dsa_probe_stream_read", "dsa_cache_flush", "dsa_probe_mfma_rate",
                   "dsa_probe_fp8_mfma", "dsa_support_last_error"]
PROBE_MFMA_FP8, PROBE_MFMA_I8, PROBE_MFMA_BF16 = 0, 1, 2
CHECK_FLAGS = {1: "seq_len", 2: "table", 4: "q_seq", 8: "q_pos", 16: "block_list"}
MOE_FP8_WORKSPACE = 0
MOE_FP4_DIRECT = 1


class PagedKVStruct(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("idx_keys", ctypes.c_void_p),
        ("idx_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
    ]


class QueriesStruct(ctypes.Structure):
    _fields_ = [
        ("num_queries", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("q_seq", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("q_idx", ctypes.c_void_p),
        ("w_idx", ctypes.c_void_p),
    ]


class MxExpertsStruct(ctypes.Structure):
    _fields_ = [
        ("w_fp4", ctypes.c_void_p),
        ("w_scale", ctypes.c_void_p),
        ("num_experts", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libdsa.so; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    kvp, qp, mxp = P(PagedKVStruct), P(QueriesStruct), P(MxExpertsStruct)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dsa_index_score": [kvp, qp, vp, vp],
        "dsa_topk_blocks": [vp, kvp, qp, i32, vp, vp, vp],
        "dsa_sparse_attn_decode": [kvp, qp, vp, vp, i32, f32, vp, vp, vp, sz, vp],
        "dsa_sparse_attn_decode_topk": [kvp, qp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp],
        "dsa_sparse_attn_prefill": [kvp, qp, vp, vp, i32, f32, vp, vp, vp],
        "dsa_sparse_decode_fused": [kvp, qp, i32, f32, vp, vp, vp, vp, vp, sz, vp],
        "dsa_sparse_decode_fused_noalloc": [kvp, qp, i32, f32, vp, vp, vp, vp, vp],
        "dsa_sparse_prefill_fused": [kvp, qp, i32, f32, vp, vp, vp, vp, vp, sz, vp],
        "dsa_index_topk": [kvp, qp, i32, vp, vp, vp, sz, vp],
        "dsa_workspace_size": [ctypes.c_int, kvp, qp, i32, P(sz)],
        "dsa_check_inputs": [kvp, qp, vp, vp, i32, vp, vp],
        "dsa_kv_write": [kvp, i32, vp, vp, vp, vp, vp],
        "dsa_index_key_write": [kvp, i32, vp, vp, vp],
        "dsa_mx_quantize": [vp, i32, i32, vp, vp, vp],
        "dsa_mxfp4_to_fp8": [mxp, vp, i32, vp, vp, vp],
        "dsa_moe_workspace_size": [mxp, i32, i32, i32, P(sz)],
        "dsa_moe_grouped_gemm": [mxp, vp, vp, i32, vp, i32, i32, vp, vp, sz, vp],
        "dsa_probe_stream_read": [vp, sz, ctypes.c_int, vp, ctypes.c_int, vp],
        "dsa_cache_flush": [vp, sz, ctypes.c_uint, vp],
        "dsa_probe_mfma_rate": [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp],
        "dsa_probe_fp8_mfma": [vp, vp, vp, ctypes.c_int, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_support_last_error.argtypes = []
    lib.dsa_support_last_error.restype = ctypes.c_char_p
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib
