"""ctypes wrapper around the fp64 CPU oracle (fd_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
and bench.py's CPU-baseline leg may import this module.  The product path
(split_kv_fd_amd) never imports it, and this module imports nothing from the
product path.

The oracle computes single-query decode attention as one softmax over the
whole valid KV range in fp64 (see the header of fd_oracle.c for the formula
and the pages it follows).  Inputs are host arrays (numpy, or torch CPU
tensors) holding raw f32 / f16 / bf16 / f64 elements; they are decoded
exactly to fp64 inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (OpenMP) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """One loaded copy of the oracle library (the tests also load mutants)."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path}")
        self.path = path
        self.lib = ctypes.CDLL(path)
        f = self.lib.fdo_decode
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                              ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        self.lib.fdo_decode_f16.restype = ctypes.c_double
        self.lib.fdo_decode_f16.argtypes = [ctypes.c_uint16]
        self.lib.fdo_decode_bf16.restype = ctypes.c_double
        self.lib.fdo_decode_bf16.argtypes = [ctypes.c_uint16]
        self.lib.fdo_max_threads.restype = ctypes.c_int

    def max_threads(self) -> int:
        return int(self.lib.fdo_max_threads())

    def decode(self, q, k, v, scale, *, dtype=None, page_table=None, seq_lens=None,
               page_size=0, rows=None, nthreads=0):
        """Whole-softmax decode attention in fp64.

        q: [B, Hq, D]; k, v: [B, Hkv, T, D] (contiguous) or pools
        [num_pages, Hkv, P, D] with page_table [B, max_pages] int32 (paged).
        seq_lens: [B] int32 valid lengths (None: all T).  For paged input T is
        taken as max_pages * page_size unless seq_lens bounds it.
        rows: optional list of flat b*Hq+h indices to compute.
        Returns (out, lse) as float64 arrays: [B, Hq, D] and [B, Hq], or
        [n_rows, D] and [n_rows] when rows is given.
        """
        qa, dt = _host_array(q, dtype)
        ka, _ = _host_array(k, dt)
        va, _ = _host_array(v, dt)
        B, Hq, D = qa.shape
        if page_table is None:
            _, Hkv, T, D2 = ka.shape
            pt = None
            max_pages = 0
        else:
            _, Hkv, P, D2 = ka.shape
            pt = np.ascontiguousarray(_to_numpy(page_table), dtype=np.int32)
            max_pages = pt.shape[1]
            if page_size == 0:
                page_size = P
            assert page_size == P
            T = max_pages * page_size
        assert D2 == D and ka.shape == va.shape
        sl = None
        if seq_lens is not None:
            sl = np.ascontiguousarray(_to_numpy(seq_lens), dtype=np.int32)
            if page_table is not None:
                T = int(max(1, min(T, sl.max())))
        rw = None
        n_rows = 0
        if rows is not None:
            rw = np.ascontiguousarray(np.asarray(rows), dtype=np.int32)
            n_rows = rw.size
            out = np.zeros((n_rows, D), np.float64)
            lse = np.zeros((n_rows,), np.float64)
        else:
            out = np.zeros((B, Hq, D), np.float64)
            lse = np.zeros((B, Hq), np.float64)
        rc = self.lib.fdo_decode(
            qa.ctypes.data, ka.ctypes.data, va.ctypes.data, DTYPE_CODE[dt],
            None if pt is None else pt.ctypes.data,
            None if sl is None else sl.ctypes.data,
            int(page_size), int(max_pages), int(B), int(Hq), int(Hkv), int(T), int(D),
            float(scale), None if rw is None else rw.ctypes.data, int(n_rows),
            out.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle rejected its arguments (code {rc})")
        return out, lse

    def decode_multi(self, q, k, v, scale, *, causal=False, dtype=None, page_table=None,
                     seq_lens=None, page_size=0, nthreads=0):
        """Decode with a small batch of n_q queries per sequence, in fp64.

        The dupenodi guide ("FlashDecoding and split-KV", opening section)
        describes decode as one query, or a small batch of queries, against
        a long KV cache.  q is [B, n_q, Hq, D]; query i of sequence b attends
        to tokens 0 .. L - 1 of the sequence's cache with L = T_b, or, when
        causal, L = T_b - (n_q - 1 - i) clamped at 0: the queries are the
        sequence's last n_q tokens (already in the cache, as when a draft of
        n_q tokens is verified), each seeing itself and the tokens before it.
        Every query is one plain decode over its own length.

        Returns out [B, n_q, Hq, D] and lse [B, n_q, Hq] (float64).
        """
        qa, dt = _host_array(q, dtype)
        B, nq, Hq, D = qa.shape
        if seq_lens is None:
            assert page_table is None, "paged caches need seq_lens"
            lens = np.full(B, _host_array(k, dt)[0].shape[2], np.int64)
        else:
            lens = np.ascontiguousarray(_to_numpy(seq_lens), dtype=np.int64)
        out = np.zeros((B, nq, Hq, D), np.float64)
        lse = np.zeros((B, nq, Hq), np.float64)
        for i in range(nq):
            li = np.maximum(lens - (nq - 1 - i), 0) if causal else lens
            o, l = self.decode(np.ascontiguousarray(qa[:, i]), k, v, scale, dtype=dt,
                               page_table=page_table, seq_lens=li.astype(np.int32),
                               page_size=page_size, nthreads=nthreads)
            out[:, i] = o
            lse[:, i] = l
        return out, lse

    def append_decode(self, q, k_new, v_new, k, v, scale, seq_lens, *, dtype=None,
                      page_table=None, page_size=0, rows=None, nthreads=0):
        """Append the step's new key and value rows to the cache, then decode
        over the grown sequence, in fp64.

        This is the fused append-KV step a serving engine runs per decode
        token (dupenodi guide "FlashDecoding and split-KV", "Walking through
        it", lists fused append-KV paths beside paged layouts and GQA): with
        T_b = seq_lens[b] tokens already cached, the rows k_new[b, j, :] and
        v_new[b, j, :] become token T_b of every kv head j, and attention
        runs over tokens 0 .. T_b (T_b + 1 of them).

        Storage slot of token T_b: K[b, j, T_b, :] of a contiguous cache
        (when T_b < T), or row T_b % P of page page_table[b, T_b // P] of a
        paged pool (when T_b // P < max_pages; that page id must be in the
        pool).  A sequence whose cache is full (T_b = T, or T_b = max_pages *
        P) has no slot: it still attends to its new token, and its cache is
        left unchanged.

        Returns (out, lse, k_after, v_after): the fp64 results as decode()
        gives them, and host copies of the caches after the store (raw
        elements, same dtype and layout as k, v).
        """
        qa, dt = _host_array(q, dtype)
        kn, _ = _host_array(k_new, dt)
        vn, _ = _host_array(v_new, dt)
        ka = _host_array(k, dt)[0].copy()
        va = _host_array(v, dt)[0].copy()
        sl = np.ascontiguousarray(_to_numpy(seq_lens), dtype=np.int64)
        B = qa.shape[0]
        assert kn.shape == vn.shape == (B, ka.shape[1], ka.shape[3])
        grown = (sl + 1).astype(np.int32)
        if page_table is None:
            T = ka.shape[2]
            # attention reads a cache one token longer, so a full sequence
            # still has a place for its new token
            k_att = np.zeros(ka.shape[:2] + (T + 1,) + ka.shape[3:], ka.dtype)
            v_att = np.zeros_like(k_att)
            k_att[:, :, :T] = ka
            v_att[:, :, :T] = va
            for b in range(B):
                t = int(sl[b])
                assert 0 <= t <= T, "seq_lens must lie in [0, T]"
                k_att[b, :, t] = kn[b]
                v_att[b, :, t] = vn[b]
                if t < T:
                    ka[b, :, t] = kn[b]
                    va[b, :, t] = vn[b]
            out, lse = self.decode(qa, k_att, v_att, scale, dtype=dt, seq_lens=grown,
                                   rows=rows, nthreads=nthreads)
            return out, lse, ka, va
        pt = np.ascontiguousarray(_to_numpy(page_table), dtype=np.int64)
        num_pages, _, P, _ = ka.shape
        if page_size:
            assert page_size == P
        max_pages = pt.shape[1]
        # attention: the stored pool plus one spare page per sequence that
        # has no slot, and a table one column wider
        pt_att = np.zeros((B, max_pages + 1), np.int32)
        pt_att[:, :max_pages] = pt
        spare = []
        for b in range(B):
            t = int(sl[b])
            assert 0 <= t <= max_pages * P, "seq_lens must lie in [0, max_pages * page_size]"
            col = t // P
            if col < max_pages:
                assert 0 <= pt[b, col] < num_pages, "the page of the new token must be in the pool"
                ka[pt[b, col], :, t % P] = kn[b]
                va[pt[b, col], :, t % P] = vn[b]
            else:
                spare.append(b)
                pt_att[b, col] = num_pages + len(spare) - 1
        k_att = np.concatenate([ka, np.zeros((len(spare),) + ka.shape[1:], ka.dtype)])
        v_att = np.concatenate([va, np.zeros((len(spare),) + va.shape[1:], va.dtype)])
        for i, b in enumerate(spare):
            t = int(sl[b])
            k_att[num_pages + i, :, t % P] = kn[b]
            v_att[num_pages + i, :, t % P] = vn[b]
        out, lse = self.decode(qa, k_att, v_att, scale, dtype=dt, page_table=pt_att,
                               seq_lens=grown, rows=rows, nthreads=nthreads)
        return out, lse, ka, va

    def decode_f16_bits(self, bits: int) -> float:
        return float(self.lib.fdo_decode_f16(bits))

    def decode_bf16_bits(self, bits: int) -> float:
        return float(self.lib.fdo_decode_bf16(bits))


def _to_numpy(x):
    if isinstance(x, np.ndarray):
        return x
    import torch  # only for host tensors handed in by the tests
    assert isinstance(x, torch.Tensor) and x.device.type == "cpu"
    return x.contiguous().numpy()


def _host_array(x, dtype):
    """Return (contiguous numpy array holding raw elements, dtype tag)."""
    if isinstance(x, np.ndarray):
        if dtype is None:
            dtype = {np.dtype(np.float32): "f32", np.dtype(np.float16): "f16",
                     np.dtype(np.float64): "f64"}[x.dtype]
        want = {"f32": np.float32, "f16": np.float16, "f64": np.float64,
                "bf16": np.uint16}[dtype]
        if dtype == "bf16":
            assert x.dtype in (np.uint16, np.int16), "bf16 arrays are passed as raw 16-bit words"
            return np.ascontiguousarray(x).view(np.uint16), dtype
        return np.ascontiguousarray(x, dtype=want), dtype
    import torch
    assert isinstance(x, torch.Tensor) and x.device.type == "cpu"
    tag = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
           torch.float64: "f64"}[x.dtype]
    if dtype is not None:
        assert dtype == tag, f"mixed dtypes {dtype} vs {tag}"
    x = x.contiguous()
    if tag == "bf16":
        return x.view(torch.int16).numpy().view(np.uint16), tag
    return x.numpy(), tag


_default = None


def default() -> Oracle:
    """The oracle built from fd_oracle.c in this directory."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default
