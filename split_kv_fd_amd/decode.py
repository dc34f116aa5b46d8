"""Torch-facing convenience over the libfd binding.

Checks shapes and devices, allocates the fp32 outputs and the workspace with
torch (device memory is torch's job here), passes raw pointers and torch's
current HIP stream to fd_decode, and raises FDError on a failing status.
No arithmetic of the decode happens in Python.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import fd

_DTYPE = {torch.float32: fd.FD_F32, torch.float16: fd.FD_F16, torch.bfloat16: fd.FD_BF16}
_PATH = {None: fd.FD_PATH_AUTO, "auto": fd.FD_PATH_AUTO, "valu": fd.FD_PATH_VALU,
         "mfma": fd.FD_PATH_MFMA, "prefill": fd.FD_PATH_PREFILL}


class FDError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fd.fd_status_string(status)}: {fd.fd_last_error()}")
        self.status = status


def make_options(dtype: torch.dtype, *, page_size: int = 0, max_pages: int = 0,
                 num_pages: int = 0, workspace: Optional[torch.Tensor] = None,
                 stream: Optional[int] = None, num_cus: int = 0,
                 path: Optional[str] = None, fused_merge: Optional[bool] = None,
                 append: bool = False, n_queries: int = 1, causal: bool = False) -> fd.fd_options_t:
    opt = fd.fd_options_t()
    fd.fd_options_init(opt)
    opt.dtype = _DTYPE[dtype]
    opt.page_size = page_size
    opt.max_pages_per_seq = max_pages
    opt.num_pages = num_pages
    opt.num_cus = num_cus
    opt.path = _PATH[path]
    # None: the library chooses; True / False force the fused merge / the
    # combine kernel.
    opt.flags = {None: 0, True: fd.FD_FLAG_FUSED_MERGE, False: fd.FD_FLAG_COMBINE_KERNEL}[fused_merge]
    if append:
        opt.flags |= fd.FD_FLAG_APPEND
    opt.n_queries = n_queries
    opt.causal = 1 if causal else 0
    if workspace is not None:
        opt.workspace = workspace.data_ptr()
        opt.workspace_bytes = workspace.numel() * workspace.element_size()
    opt.stream = stream
    return opt


def plan(B, Hq, Hkv, T, D, n_splits=0, *, dtype=torch.bfloat16, page_size=0, max_pages=0,
         num_pages=1, num_cus=0, path=None, fused_merge=None, append=False, n_queries=1,
         causal=False) -> dict:
    """What fd_decode (fd_append_decode with append=True) would launch for
    these arguments (host only)."""
    opt = make_options(dtype, page_size=page_size, max_pages=max_pages,
                       num_pages=num_pages if page_size else 0, num_cus=num_cus, path=path,
                       fused_merge=fused_merge, append=append, n_queries=n_queries, causal=causal)
    p = fd.fd_plan_t()
    st = fd.fd_plan(B, Hq, Hkv, T, D, n_splits, opt, p)
    if st != fd.FD_OK:
        raise FDError(st, "fd_plan")
    return p.as_dict()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


class Decoder:
    """A prepared decode call: validated shapes, plan, outputs and workspace.

    Calling it launches fd_decode (or the two passes separately) on torch's
    current stream; given k_new and v_new ([B, Hkv, D]) it launches
    fd_append_decode instead, which also stores them into k, v.  The
    benchmark and tests use it to keep allocation out of the timed region.
    num_cus (0: the device's own count) plans and launches as if the device
    had that many compute units.
    """

    def __init__(self, q, k, v, *, scale: Optional[float] = None, page_table=None,
                 seq_lens=None, T: Optional[int] = None, n_splits: int = 0,
                 path: Optional[str] = None, fused_merge: Optional[bool] = None, out=None, lse=None,
                 want_lse: bool = True, k_new=None, v_new=None, causal: bool = False,
                 num_cus: int = 0):
        if q.device.type != "cuda":
            raise ValueError("q, k and v must be GPU tensors")
        if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
            raise ValueError(f"q, k, v must share one of {list(_DTYPE)}; got {q.dtype}, {k.dtype}, {v.dtype}")
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not t.is_contiguous() or t.device != q.device:
                raise ValueError(f"{name} must be contiguous and on {q.device}")
        if q.dim() not in (3, 4) or k.dim() != 4 or k.shape != v.shape:
            raise ValueError("expected q [B, Hq, D] or [B, n_q, Hq, D] and k, v [B, Hkv, T, D] "
                             "or [pages, Hkv, P, D]")
        # q [B, n_q, Hq, D]: n_q queries per sequence against one cache
        self.n_queries = q.shape[1] if q.dim() == 4 else 1
        B, Hq, D = q.shape[0], q.shape[-2], q.shape[-1]
        Hkv = k.shape[1]
        if k.shape[3] != D:
            raise ValueError(f"head size mismatch: q has {D}, k has {k.shape[3]}")
        self.paged = page_table is not None
        page_size = max_pages = num_pages = 0
        if self.paged:
            if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != B:
                raise ValueError("page_table must be int32 [B, max_pages]")
            if not page_table.is_contiguous() or page_table.device != q.device:
                raise ValueError("page_table must be contiguous and on the GPU")
            num_pages, _, page_size, _ = k.shape
            max_pages = page_table.shape[1]
            T = T if T is not None else max_pages * page_size
        else:
            if k.shape[0] != B:
                raise ValueError("k, v batch differs from q")
            if T is not None and T != k.shape[2]:
                raise ValueError("T must equal the cache length for contiguous caches")
            T = k.shape[2]
        if seq_lens is not None:
            if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or seq_lens.device != q.device:
                raise ValueError("seq_lens must be int32 [B] on the GPU")
        self.append = k_new is not None
        if self.append:
            if v_new is None:
                raise ValueError("k_new and v_new go together")
            for name, t in (("k_new", k_new), ("v_new", v_new)):
                if t.shape != (B, Hkv, D) or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
                    raise ValueError(f"{name} must be a contiguous {q.dtype} [B, Hkv, D] tensor on {q.device}")
        self.new = (k_new, v_new)
        self.scale = float(1.0 / math.sqrt(D)) if scale is None else float(scale)
        self.args = (B, Hq, Hkv, T, D)
        self.n_splits = n_splits
        self.inputs = (q, k, v, page_table, seq_lens)
        self.opt = make_options(q.dtype, page_size=page_size, max_pages=max_pages,
                                num_pages=num_pages, path=path, fused_merge=fused_merge,
                                append=self.append, n_queries=self.n_queries, causal=causal,
                                num_cus=num_cus)
        p = fd.fd_plan_t()
        st = fd.fd_plan(B, Hq, Hkv, T, D, n_splits, self.opt, p)
        if st != fd.FD_OK:
            raise FDError(st, "fd_plan")
        self.plan = p.as_dict()
        self.workspace = None
        if p.workspace_bytes:
            self.workspace = torch.empty(p.workspace_bytes, dtype=torch.uint8, device=q.device)
            self.opt.workspace = self.workspace.data_ptr()
            self.opt.workspace_bytes = p.workspace_bytes
        rows = (B, self.n_queries, Hq) if q.dim() == 4 else (B, Hq)
        self.out = out if out is not None else torch.empty(rows + (D,), dtype=torch.float32, device=q.device)
        self.lse = lse if lse is not None else (
            torch.empty(rows, dtype=torch.float32, device=q.device) if want_lse else None)

    def _call(self, fn, name):
        q, k, v, pt, sl = self.inputs
        self.opt.stream = torch.cuda.current_stream(q.device).cuda_stream
        B, Hq, Hkv, T, D = self.args
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(pt), _ptr(sl), _ptr(self.out), _ptr(self.lse),
                B, Hq, Hkv, T, D, self.scale, self.n_splits, self.opt)
        if st != fd.FD_OK:
            raise FDError(st, name)

    def __call__(self):
        """fd_decode (or fd_append_decode): split pass and, if planned, the
        combine pass."""
        if self.append:
            q, k, v, pt, sl = self.inputs
            self.opt.stream = torch.cuda.current_stream(q.device).cuda_stream
            B, Hq, Hkv, T, D = self.args
            kn, vn = self.new
            st = fd.fd_append_decode(_ptr(q), _ptr(kn), _ptr(vn), _ptr(k), _ptr(v), _ptr(pt),
                                     _ptr(sl), _ptr(self.out), _ptr(self.lse), B, Hq, Hkv, T, D,
                                     self.scale, self.n_splits, self.opt)
            if st != fd.FD_OK:
                raise FDError(st, "fd_append_decode")
            return self.out, self.lse
        self._call(fd.fd_decode, "fd_decode")
        return self.out, self.lse

    def split(self):
        """fd_split alone."""
        self._call(fd.fd_split, "fd_split")

    def combine(self):
        """fd_combine alone (no-op for a one-split plan)."""
        q = self.inputs[0]
        self.opt.stream = torch.cuda.current_stream(q.device).cuda_stream
        B, Hq, Hkv, T, D = self.args
        st = fd.fd_combine(_ptr(self.inputs[4]), _ptr(self.out), _ptr(self.lse), B, Hq, Hkv, T, D,
                           self.n_splits, self.opt)
        if st != fd.FD_OK:
            raise FDError(st, "fd_combine")


def decode(q, k, v, *, scale=None, page_table=None, seq_lens=None, T=None, n_splits=0,
           path=None, fused_merge=None, causal=False):
    """out [B, Hq, D] fp32 and lse [B, Hq] fp32 of single-query decode
    attention; with q [B, n_q, Hq, D] (several queries per sequence, causal
    or not), out [B, n_q, Hq, D] and lse [B, n_q, Hq]."""
    return Decoder(q, k, v, scale=scale, page_table=page_table, seq_lens=seq_lens, T=T,
                   n_splits=n_splits, path=path, fused_merge=fused_merge, causal=causal)()


def append_decode(q, k_new, v_new, k, v, *, seq_lens, scale=None, page_table=None, T=None,
                  n_splits=0, path=None, fused_merge=None):
    """Store k_new, v_new [B, Hkv, D] as token seq_lens[b] of each sequence's
    cache (k, v are updated in place), then decode over seq_lens[b] + 1
    tokens: out [B, Hq, D] fp32 and lse [B, Hq] fp32."""
    return Decoder(q, k, v, scale=scale, page_table=page_table, seq_lens=seq_lens, T=T,
                   n_splits=n_splits, path=path, fused_merge=fused_merge, k_new=k_new,
                   v_new=v_new)()
