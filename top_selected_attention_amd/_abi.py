"""ctypes mirror of include/top_selected_attention.h (structs, codes, signatures)."""

import ctypes
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

BF16, FP16 = 0, 1
LAYOUT_BNSD, LAYOUT_TND, LAYOUT_BSND = 0, 1, 2

STATUS = {
    0: "TSA_OK", 1: "TSA_ERR_NULL", 2: "TSA_ERR_INVALID", 3: "TSA_ERR_UNSUPPORTED",
    4: "TSA_ERR_WORKSPACE", 5: "TSA_ERR_HIP", 6: "TSA_ERR_DATA", 7: "TSA_ERR_SCRATCH",
}

EXPORTS = [
    "tsa_status_string", "tsa_args_sizeof",
    "bsa_fwd_workspace_size", "bsa_fwd", "bsa_bwd_workspace_size", "bsa_bwd",
    "bsa_compact_workspace_size", "bsa_compact",
    "nsa_select_fwd_workspace_size", "nsa_select_fwd", "nsa_select_bwd_workspace_size",
    "nsa_select_bwd", "nsa_compact_blocks_total", "nsa_compact_workspace_size", "nsa_compact",
    "sfa_paged_fwd_workspace_size", "sfa_paged_fwd",
    "sfa_paged_fwd_noalloc_max_bytes", "sfa_paged_fwd_noalloc",
    "sfa_sharedkv_fwd_workspace_size", "sfa_sharedkv_fwd",
    "sfa_sharedkv_metadata_size", "sfa_sharedkv_metadata",
    "floyd_fwd_workspace_size", "floyd_fwd", "floyd_bwd_workspace_size", "floyd_bwd",
]


# reuse_lists, n_events, events: the common tail of every args struct
TRAIL = [("reuse_lists", c_int32), ("n_events", c_int32), ("events", POINTER(c_void_p))]


class TsaError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


class BsaFwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("q_layout", c_int32), ("kv_layout", c_int32),
        ("B", c_int32), ("N1", c_int32), ("N2", c_int32), ("Sq", c_int32), ("Skv", c_int32),
        ("D", c_int32), ("block_q", c_int32), ("block_kv", c_int32), ("sparse_mode", c_int32),
        ("scale", c_float), ("validate", c_int32),
        ("block_mask", c_void_p), ("q", c_void_p), ("k", c_void_p), ("v", c_void_p),
        ("out", c_void_p), ("lse", c_void_p),
    ] + TRAIL + [("cu_seqlens_q", POINTER(c_int32)), ("cu_seqlens_kv", POINTER(c_int32)),
                 ("atten_mask", c_void_p), ("atten_mask_stride_b", c_int64),
                 ("atten_mask_stride_n", c_int64)]


class BsaBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("q_layout", c_int32), ("kv_layout", c_int32),
        ("B", c_int32), ("N1", c_int32), ("N2", c_int32), ("Sq", c_int32), ("Skv", c_int32),
        ("D", c_int32), ("block_q", c_int32), ("block_kv", c_int32), ("sparse_mode", c_int32),
        ("scale", c_float), ("validate", c_int32),
        ("block_mask", c_void_p), ("q", c_void_p), ("k", c_void_p), ("v", c_void_p),
        ("out", c_void_p), ("dout", c_void_p), ("lse", c_void_p),
        ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p),
    ] + TRAIL + [("cu_seqlens_q", POINTER(c_int32)), ("cu_seqlens_kv", POINTER(c_int32)),
                 ("atten_mask", c_void_p), ("atten_mask_stride_b", c_int64),
                 ("atten_mask_stride_n", c_int64)]


_NSA_COMMON = [
    ("dtype", c_int32), ("layout", c_int32), ("B", c_int32), ("T", c_int32), ("Tk", c_int32),
    ("N1", c_int32), ("N2", c_int32), ("D", c_int32), ("Dv", c_int32),
    ("cu_seqlens_q", POINTER(c_int32)), ("cu_seqlens_kv", POINTER(c_int32)),
    ("sbs", c_int32), ("sbc", c_int32), ("sparse_mode", c_int32), ("scale", c_float),
    ("validate", c_int32), ("topk", c_void_p), ("q", c_void_p), ("k", c_void_p),
    ("v", c_void_p),
]


class NsaFwdArgs(ctypes.Structure):
    _fields_ = _NSA_COMMON + [("out", c_void_p), ("lse", c_void_p)] + TRAIL


class NsaBwdArgs(ctypes.Structure):
    _fields_ = _NSA_COMMON + [
        ("out", c_void_p), ("dout", c_void_p), ("lse", c_void_p),
        ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p),
    ] + TRAIL


class SfaArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("q_layout", c_int32), ("B", c_int32), ("Sq", c_int32),
        ("N1", c_int32), ("N2", c_int32), ("D", c_int32), ("Dr", c_int32), ("Dv", c_int32),
        ("num_pages", c_int32), ("page_size", c_int32), ("max_pages", c_int32),
        ("topk", c_int32), ("sparse_block_size", c_int32), ("sparse_mode", c_int32),
        ("scale", c_float), ("validate", c_int32),
        ("q", c_void_p), ("q_rope", c_void_p), ("key_cache", c_void_p),
        ("key_rope_cache", c_void_p), ("value_cache", c_void_p),
        ("block_table", c_void_p), ("kv_lens", c_void_p), ("topk_indices", c_void_p),
        ("out", c_void_p), ("lse", c_void_p),
    ] + TRAIL + [("T", c_int32), ("cu_seqlens_q", POINTER(c_int32))]


class SfaSharedkvArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("q_layout", c_int32), ("B", c_int32), ("Sq", c_int32),
        ("T", c_int32), ("N1", c_int32), ("N2", c_int32), ("D", c_int32), ("Dr", c_int32),
        ("scale", c_float), ("q", c_void_p), ("q_rope", c_void_p),
        ("cu_seqlens_q", POINTER(c_int32)), ("seqused_kv", c_void_p),
        ("has_ori_kv", c_int32), ("has_cmp_kv", c_int32),
        ("ori_win_left", c_int32), ("ori_win_right", c_int32),
        ("ori_num_pages", c_int32), ("ori_page_size", c_int32), ("ori_max_pages", c_int32),
        ("ori_key_cache", c_void_p), ("ori_key_rope_cache", c_void_p),
        ("ori_block_table", c_void_p),
        ("cmp_ratio", c_int32), ("cmp_topk", c_int32),
        ("cmp_num_pages", c_int32), ("cmp_page_size", c_int32), ("cmp_max_pages", c_int32),
        ("cmp_key_cache", c_void_p), ("cmp_key_rope_cache", c_void_p),
        ("cmp_block_table", c_void_p), ("cmp_topk_indices", c_void_p),
        ("out", c_void_p), ("lse", c_void_p), ("tasks", c_void_p),
    ] + TRAIL


_FLOYD_COMMON = [
    ("dtype", c_int32), ("B", c_int32), ("H", c_int32), ("N", c_int32), ("M", c_int32),
    ("K", c_int32), ("D", c_int32), ("scale", c_float),
    ("q", c_void_p), ("k1", c_void_p), ("v1", c_void_p), ("k2", c_void_p), ("v2", c_void_p),
]


class FloydFwdArgs(ctypes.Structure):
    _fields_ = _FLOYD_COMMON + [("out", c_void_p), ("lse", c_void_p)] + TRAIL


class FloydBwdArgs(ctypes.Structure):
    _fields_ = _FLOYD_COMMON + [
        ("out", c_void_p), ("dout", c_void_p), ("lse", c_void_p),
        ("dq", c_void_p), ("dk1", c_void_p), ("dv1", c_void_p), ("dk2", c_void_p),
        ("dv2", c_void_p),
    ] + TRAIL


ARG_STRUCTS = [BsaFwdArgs, BsaBwdArgs, NsaFwdArgs, NsaBwdArgs, SfaArgs, SfaSharedkvArgs,
               FloydFwdArgs, FloydBwdArgs]

_lib = None


def load(path):
    """dlopen the library and declare every export's signature."""
    global _lib
    lib = ctypes.CDLL(path)
    lib.tsa_status_string.restype = c_char_p
    lib.tsa_status_string.argtypes = [c_int]
    lib.tsa_args_sizeof.restype = c_size_t
    lib.tsa_args_sizeof.argtypes = [c_int]
    P = c_void_p
    sig = {
        "bsa_fwd_workspace_size": [P, P], "bsa_fwd": [P, P, c_size_t, P],
        "bsa_bwd_workspace_size": [P, P], "bsa_bwd": [P, P, c_size_t, P],
        "bsa_compact_workspace_size": [P, P],
        "bsa_compact": [P, P, P, P, P, P, c_size_t, P],
        "nsa_select_fwd_workspace_size": [P, P], "nsa_select_fwd": [P, P, c_size_t, P],
        "nsa_select_bwd_workspace_size": [P, P], "nsa_select_bwd": [P, P, c_size_t, P],
        "nsa_compact_blocks_total": [P, P], "nsa_compact_workspace_size": [P, P],
        "nsa_compact": [P, P, P, P, P, P, c_size_t, P],
        "sfa_paged_fwd_workspace_size": [P, P], "sfa_paged_fwd": [P, P, c_size_t, P],
        "sfa_paged_fwd_noalloc": [P, P],
        "sfa_sharedkv_fwd_workspace_size": [P, P], "sfa_sharedkv_fwd": [P, P, c_size_t, P],
        "sfa_sharedkv_metadata_size": [P, P], "sfa_sharedkv_metadata": [P, P, c_size_t, P],
        "floyd_fwd_workspace_size": [P, P], "floyd_fwd": [P, P, c_size_t, P],
        "floyd_bwd_workspace_size": [P, P], "floyd_bwd": [P, P, c_size_t, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = args
    lib.sfa_paged_fwd_noalloc_max_bytes.restype = c_size_t
    lib.sfa_paged_fwd_noalloc_max_bytes.argtypes = []
    for i, s in enumerate(ARG_STRUCTS):
        n = lib.tsa_args_sizeof(i)
        if n != ctypes.sizeof(s):
            raise ImportError(f"ABI mismatch: {s.__name__} is {ctypes.sizeof(s)} bytes here, "
                              f"{n} in the library")
    _lib = lib
    return lib


def call(fn, *args):
    s = fn(*args)
    if s != 0:
        raise TsaError(s, _lib.tsa_status_string(s).decode())
    return s
