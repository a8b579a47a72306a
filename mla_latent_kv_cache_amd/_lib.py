"""ctypes declarations of the C ABI in include/mla.h and loading of the in-tree library."""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LATENT_LIB names another build of the same library (the host-sanitized one of the CPU test suite)
LIB_PATH = os.environ.get("MLA_LATENT_LIB") or os.path.join(PKG, "libmla_latent.so")

MLA_OK = 0
MLA_F32, MLA_BF16 = 0, 1
MLA_CACHE_DENSE, MLA_CACHE_INT4_G32, MLA_CACHE_INT2_G32_WIN, MLA_CACHE_INT4_G32_WIN = 0, 1, 2, 3

EXPORTED = [
    "mla_cache_append",
    "mla_cache_append_workspace_bytes",
    "mla_cache_append_ws",
    "mla_decode_workspace_bytes",
    "mla_decode",
    "mla_decode_phase",
    "mla_decode_multi_workspace_bytes",
    "mla_decode_multi",
    "mla_decode_step_workspace_bytes",
    "mla_decode_step",
    "mla_decode_step_static",
    "mla_decode_step_phase",
    "mla_prefill_workspace_bytes",
    "mla_prefill",
    "mla_quantize_int4",
    "mla_quantize_int2",
    "mla_rope_tables",
    "mla_status_string",
]


class MlaConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32)
                for n in ("d_model", "n_heads", "d_head", "r_pairs", "d_kv", "dtype", "cache_fmt", "rope_heads")]


class MlaWeights(ctypes.Structure):
    _fields_ = [
        ("w_dkv", ctypes.c_void_p),
        ("w_krope", ctypes.c_void_p),
        ("w_uk", ctypes.c_void_p),
        ("w_uv", ctypes.c_void_p),
        ("pair_idx", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p),
        ("rope_len", ctypes.c_int32),
    ]


class MlaCache(ctypes.Structure):
    _fields_ = [
        ("ckv", ctypes.c_void_p),
        ("ckv_scale", ctypes.c_void_p),
        ("krope", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("t_max", ctypes.c_int32),
        ("ckv_window", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libmla_latent.so (after torch, so that torch's HIP runtime is the one both use)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (brings in the HIP runtime the library binds to)

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first (python -m mla_latent_kv_cache_amd.build)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    C, W, K = ctypes.POINTER(MlaConfig), ctypes.POINTER(MlaWeights), ctypes.POINTER(MlaCache)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mla_cache_append.argtypes = [C, W, K, P, P, i32, i32, P]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_cache_append_workspace_bytes.argtypes = [C, i32, i32]
    lib.mla_cache_append_workspace_bytes.restype = sz
    lib.mla_cache_append_ws.argtypes = [C, W, K, P, P, i32, i32, P, sz, P]
    lib.mla_cache_append_ws.restype = ctypes.c_int
    lib.mla_decode_workspace_bytes.argtypes = [C, i32, i32]
    lib.mla_decode_workspace_bytes.restype = sz
    lib.mla_decode.argtypes = [C, W, K, P, P, i32, P, P, sz, P]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode_phase.argtypes = [ctypes.c_int, C, W, K, P, P, i32, P, P, sz, P]
    lib.mla_decode_phase.restype = ctypes.c_int
    lib.mla_decode_multi_workspace_bytes.argtypes = [C, i32, i32, i32]
    lib.mla_decode_multi_workspace_bytes.restype = sz
    lib.mla_decode_multi.argtypes = [C, W, K, P, i32, P, i32, P, P, sz, P]
    lib.mla_decode_multi.restype = ctypes.c_int
    lib.mla_decode_step_workspace_bytes.argtypes = [C, i32, i32, i32]
    lib.mla_decode_step_workspace_bytes.restype = sz
    lib.mla_decode_step.argtypes = [C, W, K, P, P, i32, i32, P, P, i32, P, P, sz, P]
    lib.mla_decode_step.restype = ctypes.c_int
    lib.mla_decode_step_static.argtypes = [C, W, K, P, P, i32, i32, P, P, i32, P, P]
    lib.mla_decode_step_static.restype = ctypes.c_int
    lib.mla_decode_step_phase.argtypes = [ctypes.c_int, C, W, K, P, P, i32, i32, P, P, i32, P, P, sz, P]
    lib.mla_decode_step_phase.restype = ctypes.c_int
    lib.mla_rope_tables.argtypes = [i32, i32, ctypes.c_double, P, P]
    lib.mla_rope_tables.restype = ctypes.c_int
    lib.mla_prefill_workspace_bytes.argtypes = [C, i32, i32]
    lib.mla_prefill_workspace_bytes.restype = sz
    lib.mla_prefill.argtypes = [C, W, K, P, i32, P, P, sz, P]
    lib.mla_prefill.restype = ctypes.c_int
    lib.mla_quantize_int4.argtypes = [P, i64, P, P, P]
    lib.mla_quantize_int4.restype = ctypes.c_int
    lib.mla_quantize_int2.argtypes = [P, i64, P, P, P]
    lib.mla_quantize_int2.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib
