"""ctypes binding of libfd (include/fd.h): the same entry points, raw pointers.

Argument marshalling only -- every step of the decode runs in the HIP
library.  Importing this module does not load the library; the first call
does, and raises if libfd.so has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

# The in-tree build; FD_LIBRARY may name another build of the same sources
# (for comparing compile-time variants).
LIB_PATH = os.environ.get("FD_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfd.so")

FD_F32, FD_F16, FD_BF16 = 0, 1, 2
FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_ERR_HIP = range(5)
FD_PATH_AUTO, FD_PATH_VALU, FD_PATH_MFMA, FD_PATH_PREFILL = -1, 0, 1, 2
FD_FLAG_FUSED_MERGE = 0x1
FD_FLAG_COMBINE_KERNEL = 0x2
FD_FLAG_APPEND = 0x4

# Every function include/fd.h declares.
EXPORTS = ("fd_options_init", "fd_plan", "fd_workspace_bytes", "fd_decode", "fd_append_decode",
           "fd_split", "fd_combine", "fd_decode_noalloc", "fd_status_string", "fd_last_error")
# Bytes of the static device scratch fd_decode_noalloc uses (per GPU).
FD_NOALLOC_SCRATCH_BYTES = 32 << 20


class fd_options_t(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("path", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p), ("n_queries", ctypes.c_int32), ("causal", ctypes.c_int32)]


class fd_plan_t(ctypes.Structure):
    _fields_ = [("n_splits", ctypes.c_int32), ("chunk", ctypes.c_int32), ("path", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("heads_per_block", ctypes.c_int32),
                ("head_blocks", ctypes.c_int32), ("grid", ctypes.c_int32 * 3),
                ("block", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("fused", ctypes.c_int32), ("stream", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self) -> dict:
        return {"n_splits": self.n_splits, "chunk": self.chunk,
                "path": {0: "valu", 1: "mfma", 2: "prefill"}.get(self.path, self.path), "tile": self.tile,
                "heads_per_block": self.heads_per_block, "head_blocks": self.head_blocks,
                "grid": list(self.grid), "block": self.block, "combine": bool(self.combine),
                "fused": bool(self.fused), "stream": bool(self.stream),
                "workspace_bytes": self.workspace_bytes}


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_OPT = ctypes.POINTER(fd_options_t)


def load() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m split_kv_fd_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.fd_options_init.restype = None
        lib.fd_options_init.argtypes = [_OPT]
        lib.fd_plan.restype = _I
        lib.fd_plan.argtypes = [_I] * 6 + [_OPT, ctypes.POINTER(fd_plan_t)]
        lib.fd_workspace_bytes.restype = ctypes.c_size_t
        lib.fd_workspace_bytes.argtypes = [_I] * 6 + [_OPT]
        decode_args = [_P, _P, _P, _P, _P, _P, _P] + [_I] * 5 + [ctypes.c_float, _I, _OPT]
        for name in ("fd_decode", "fd_split", "fd_decode_noalloc"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = decode_args
        lib.fd_append_decode.restype = _I
        lib.fd_append_decode.argtypes = [_P] * 9 + [_I] * 5 + [ctypes.c_float, _I, _OPT]
        lib.fd_combine.restype = _I
        lib.fd_combine.argtypes = [_P, _P, _P] + [_I] * 6 + [_OPT]
        lib.fd_status_string.restype = ctypes.c_char_p
        lib.fd_status_string.argtypes = [_I]
        lib.fd_last_error.restype = ctypes.c_char_p
        lib.fd_last_error.argtypes = []
        _lib = lib
    return _lib


def fd_options_init(opt: fd_options_t) -> None:
    load().fd_options_init(ctypes.byref(opt))


def fd_plan(B, Hq, Hkv, T, D, n_splits, opt, plan: fd_plan_t) -> int:
    return load().fd_plan(B, Hq, Hkv, T, D, n_splits, ctypes.byref(opt), ctypes.byref(plan))


def fd_workspace_bytes(B, Hq, Hkv, T, D, n_splits, opt) -> int:
    return load().fd_workspace_bytes(B, Hq, Hkv, T, D, n_splits, ctypes.byref(opt))


def fd_decode(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
              n_splits, opt) -> int:
    return load().fd_decode(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T,
                            D, scale, n_splits, ctypes.byref(opt))


def fd_decode_noalloc(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                      n_splits, opt) -> int:
    return load().fd_decode_noalloc(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv,
                                    T, D, scale, n_splits, ctypes.byref(opt))


def fd_append_decode(q, k_new, v_new, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq,
                     Hkv, T, D, scale, n_splits, opt) -> int:
    return load().fd_append_decode(q, k_new, v_new, k_cache, v_cache, page_table, seq_lens, out,
                                   lse, B, Hq, Hkv, T, D, scale, n_splits, ctypes.byref(opt))


def fd_split(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
             n_splits, opt) -> int:
    return load().fd_split(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T,
                           D, scale, n_splits, ctypes.byref(opt))


def fd_combine(seq_lens, out, lse, B, Hq, Hkv, T, D, n_splits, opt) -> int:
    return load().fd_combine(seq_lens, out, lse, B, Hq, Hkv, T, D, n_splits, ctypes.byref(opt))


def fd_status_string(status: int) -> str:
    return load().fd_status_string(status).decode()


def fd_last_error() -> str:
    return load().fd_last_error().decode()
