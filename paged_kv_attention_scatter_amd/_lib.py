"""ctypes declarations of libpkv.so's C ABI (include/pkv.h).

The library is built in-tree by ``paged_kv_attention_scatter_amd.build``. If it
is missing, importing any compute entry point raises: there is no fallback.
"""

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

# PKV_LIB_PATH selects another build of the same library (the sanitizer
# build of the host code, for instance).
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
STATUS_NAMES = {
    0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_DTYPE", -3: "PKV_ERR_SHAPE",
    -4: "PKV_ERR_LENGTHS", -5: "PKV_ERR_ALIGN", -6: "PKV_ERR_WORKSPACE", -7: "PKV_ERR_HIP",
    -8: "PKV_ERR_DEVICE",
}
PKV_F32, PKV_BF16 = 0, 1
PKV_I32, PKV_I64 = 0, 1
PKV_PREP_ALL_GREEDY, PKV_PREP_USE_TOP_K, PKV_PREP_USE_TOP_P = 0x1, 0x2, 0x4
NOALLOC_SCRATCH_BYTES = 16 << 20  # PKV_NOALLOC_SCRATCH_BYTES
FAULT_BITS = {
    0x1: "PKV_FAULT_STORE_SLOT", 0x2: "PKV_FAULT_LENGTH", 0x4: "PKV_FAULT_TABLE_SLOT",
    0x8: "PKV_FAULT_TABLE_ROW", 0x10: "PKV_FAULT_QROWS", 0x20: "PKV_FAULT_OUT_LOC",
}


class PkvPool(ctypes.Structure):
    _fields_ = [
        ("k", c_void_p), ("v", c_void_p), ("num_slots", c_int64), ("row_stride", c_int64),
        ("kv_heads", c_int32), ("head_dim", c_int32), ("page_size", c_int32), ("dtype", c_int32),
    ]


class PkvQNormRope(ctypes.Structure):
    _fields_ = [("q_norm_weight", c_void_p), ("eps", c_float), ("rope_theta", c_float)]


_P_i32 = POINTER(c_int32)
_P_f32 = POINTER(c_float)

# name -> (restype, argtypes); every symbol include/pkv.h declares.
SIGNATURES = {
    "pkv_store_kv": (c_int32, [POINTER(PkvPool), c_void_p, c_int32, c_int64, c_void_p, c_int64,
                               c_void_p, c_int64, c_void_p]),
    "pkv_embedding_gather": (c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, c_void_p, c_int64, c_int64,
                                      c_int64, c_void_p, c_int64, c_void_p]),
    "pkv_qk_norm_rope_store_kv": (c_int32, [POINTER(PkvPool), c_void_p, c_int32, c_int64, c_void_p, c_int64,
                                           c_void_p, c_int64, c_int32, c_void_p, c_int64, c_void_p, c_int64,
                                           c_void_p, c_void_p, c_void_p, c_float, c_float, c_void_p]),
    "pkv_paged_attention_decode": (c_int32, [POINTER(PkvPool), c_void_p, c_int64, c_void_p, c_int64,
                                             c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                             c_void_p, c_void_p, c_int64, c_float, c_void_p, c_size_t,
                                             c_void_p]),
    "pkv_decode_workspace_size": (c_size_t, [c_int32, c_int32, c_int64]),
    "pkv_paged_attention_decode_store": (c_int32, [POINTER(PkvPool), c_void_p, c_int32, c_void_p, c_int64,
                                                   c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                                   c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                                   c_void_p, c_void_p, c_int64, c_float, c_void_p, c_size_t,
                                                   c_void_p]),
    "pkv_paged_attention_decode_qnr": (c_int32, [POINTER(PkvPool), c_void_p, c_int64, c_void_p, c_int64,
                                                 c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                                 c_void_p, c_void_p, c_int64, c_float, POINTER(PkvQNormRope),
                                                 c_void_p, c_size_t, c_void_p]),
    "pkv_paged_attention_extend_qnr": (c_int32, [POINTER(PkvPool), c_void_p, c_int64, c_void_p, c_int64,
                                                 c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                                 c_void_p, c_void_p, c_int64, c_int32, c_float,
                                                 POINTER(PkvQNormRope), c_void_p, c_size_t, c_void_p]),
    "pkv_paged_attention_decode_noalloc": (c_int32, [POINTER(PkvPool), c_void_p, c_int64, c_void_p, c_int64,
                                                     c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                                     c_void_p, c_void_p, c_int64, c_float, c_void_p]),
    "pkv_paged_attention_extend": (c_int32, [POINTER(PkvPool), c_void_p, c_int64, c_void_p, c_int64,
                                             c_int32, c_int32, c_void_p, c_int32, c_int64, c_void_p,
                                             c_void_p, c_void_p, c_int64, c_int32, c_float, c_void_p,
                                             c_size_t, c_void_p]),
    "pkv_extend_workspace_size": (c_size_t, [c_int32, c_int32, c_int64, c_int32]),
    "pkv_sample": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "pkv_sample_workspace_size": (c_size_t, [c_int32, c_int32]),
    "pkv_num_pages": (c_int64, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int64,
                                c_int64, c_double]),
    "pkv_prepare_sampling": (c_int32, [c_int32, _P_f32, _P_i32, _P_f32, c_int32, _P_f32, _P_i32,
                                       _P_f32, _P_i32]),
    "pkv_read_faults": (c_int32, [c_void_p, POINTER(c_uint32)]),
    "pkv_last_error": (c_char_p, []),
    "pkv_version": (c_char_p, []),
}

_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m paged_kv_attention_scatter_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode())
