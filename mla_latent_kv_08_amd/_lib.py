"""ctypes view of libmla.so: the structs and entry points of include/mla.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4

MLA_F32 = 0
MLA_BF16 = 1
MLA_FP4_E2M1_E4M3X16 = 2
MLA_ROPE_INTERLEAVED = 0
MLA_ROPE_HALVES = 1
MLA_ROPE_LATENT_TAIL = 2
MLA_NOALLOC_SCRATCH_BYTES = 40 << 20

EXPORTS = (
    "mla_absorb_q",
    "mla_decode_workspace_size",
    "mla_decode_attn",
    "mla_decode_attn_up",
    "mla_decode_attn_noalloc",
    "mla_up_proj_v",
    "mla_cache_append",
    "mla_rope_append",
    "mla_sink_inverse_rope",
    "mla_grouped_out_proj",
    "mla_prefill_attn",
    "mla_prefill_workspace_size",
    "mla_append_absorb",
    "mla_dequant_rows",
    "mla_status_string",
)


class MlaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "q_len", "d_nope", "d_rope", "d_v", "d_latent")]


class MlaKvCache(ctypes.Structure):
    _fields_ = [
        ("latent_dtype", ctypes.c_int32),
        ("rope_dtype", ctypes.c_int32),
        ("latent", ctypes.c_void_p),
        ("latent_scale", ctypes.c_void_p),
        ("rope", ctypes.c_void_p),
        ("latent_stride", ctypes.c_int64),
        ("scale_stride", ctypes.c_int64),
        ("rope_stride", ctypes.c_int64),
        ("num_rows", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("page_table_stride", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MlaDecodeOpts(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_LIB = None


def load() -> ctypes.CDLL:
    """Load libmla.so (built in-tree); raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_08_amd.build` "
            "(or __graft_entry__.build()) before using the MLA kernels")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    lib.mla_absorb_q.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, P, P]
    lib.mla_absorb_q.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [ctypes.POINTER(MlaDims), I32, I32,
                                              ctypes.POINTER(MlaDecodeOpts),
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    lib.mla_decode_attn.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, ctypes.POINTER(MlaKvCache), P,
                                    I32, ctypes.c_float, P, P, P, ctypes.c_size_t,
                                    ctypes.POINTER(MlaDecodeOpts), P]
    lib.mla_decode_attn.restype = ctypes.c_int
    lib.mla_decode_attn_up.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, ctypes.POINTER(MlaKvCache), P,
                                       I32, ctypes.c_float, P, P, P, P, P, ctypes.c_size_t,
                                       ctypes.POINTER(MlaDecodeOpts), P]
    lib.mla_decode_attn_up.restype = ctypes.c_int
    lib.mla_decode_attn_noalloc.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, ctypes.POINTER(MlaKvCache), P,
                                            I32, ctypes.c_float, P, P, ctypes.POINTER(MlaDecodeOpts), P]
    lib.mla_decode_attn_noalloc.restype = ctypes.c_int
    lib.mla_up_proj_v.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, P]
    lib.mla_up_proj_v.restype = ctypes.c_int
    lib.mla_cache_append.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, ctypes.POINTER(MlaKvCache), P, P]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_rope_append.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, P, I32, I32, ctypes.POINTER(MlaKvCache),
                                    P, P]
    lib.mla_rope_append.restype = ctypes.c_int
    lib.mla_sink_inverse_rope.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, P, P, I32, I32, P, P]
    lib.mla_sink_inverse_rope.restype = ctypes.c_int
    lib.mla_grouped_out_proj.argtypes = [ctypes.POINTER(MlaDims), I32, I32, I32, P, P, P, P]
    lib.mla_grouped_out_proj.restype = ctypes.c_int
    lib.mla_prefill_attn.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, ctypes.POINTER(MlaKvCache), P, P,
                                     ctypes.c_float, P, P, P, ctypes.c_size_t, P]
    lib.mla_prefill_workspace_size.argtypes = [ctypes.POINTER(MlaDims), I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_workspace_size.restype = ctypes.c_int
    lib.mla_prefill_attn.restype = ctypes.c_int
    lib.mla_append_absorb.argtypes = [ctypes.POINTER(MlaDims), I32, P, P, ctypes.POINTER(MlaKvCache), P,
                                      I32, P, P, P, P, P]
    lib.mla_append_absorb.restype = ctypes.c_int
    lib.mla_dequant_rows.argtypes = [ctypes.POINTER(MlaKvCache), I32, P, I32, P, P]
    lib.mla_dequant_rows.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().mla_status_string(int(status)).decode()
    except RuntimeError:
        return "libmla.so not loaded"


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, where)
