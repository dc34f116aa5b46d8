"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
host copies of the same inputs, and compare with the stated tolerances.

Tolerances (on max |out_gpu - out_oracle| / max |V| over the valid tokens):
1e-5 for fp32 K/V and 2e-3 for f16/bf16 K/V with fp32 accumulation; lse
within 1e-4 (fp32) / 1e-3 (f16, bf16) absolute.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as oracle_mod
from split_kv_fd_amd.decode import Decoder

OUT_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
LSE_TOL = {"f32": 1e-4, "f16": 1e-3, "bf16": 1e-3}


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(case, n_splits=0, path=None, scale=None, fused_merge=None, poison=False):
    q, k, v = case.q, case.k, case.v
    dec = Decoder(q, k, v, scale=case.spec.scale if scale is None else scale,
                  page_table=case.page_table, seq_lens=case.seq_lens,
                  T=case.spec.T if case.page_table is not None else None,
                  n_splits=n_splits, path=path, fused_merge=fused_merge)
    if poison and dec.workspace is not None:
        dec.workspace.fill_(0xFF)          # NaN partials, foreign counter tags
    announce(f"decode {case.spec.name} B={case.spec.B} Hq={case.spec.Hq} Hkv={case.spec.Hkv} "
             f"T={case.spec.T} D={case.spec.D} {case.spec.dtype} seed={case.spec.seed} "
             f"n_splits={n_splits} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy(), dec.plan


def max_abs_v(case, b=None) -> float:
    """max |V| over the valid tokens (of sequence b, or all)."""
    lens = case.lengths()
    v = case.v
    if case.page_table is None:
        bs = range(case.spec.B) if b is None else [b]
        return max(float(v[bb, :, :lens[bb]].abs().max()) if lens[bb] else 0.0 for bb in bs)
    P = case.spec.page_size
    bs = range(case.spec.B) if b is None else [b]
    m = 0.0
    for bb in bs:
        n = -(-lens[bb] // P)
        if n == 0:
            continue
        pages = case.page_table[bb, :n].long()
        blk = v[pages]                                   # [n, Hkv, P, D]
        blk = blk.transpose(1, 2).reshape(n * P, case.spec.Hkv, case.spec.D)[:lens[bb]]
        m = max(m, float(blk.abs().max()))
    return m


def oracle_full(case):
    c = case.to("cpu")
    return oracle_mod.default().decode(c.q, c.k, c.v, case.spec.scale, page_table=c.page_table,
                                       seq_lens=c.seq_lens)


def compare(case, out, lse, ref_out, ref_lse, vmax, what=""):
    tol = OUT_TOL[case.spec.dtype]
    ltol = LSE_TOL[case.spec.dtype]
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = float(np.max(np.abs(out - ref_out))) / max(vmax, 1e-30)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: lse finiteness differs"
    assert np.all(lse[~fin] == ref_lse[~fin]), f"{what}: lse infinities differ"
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0.0))
    announce(f"{what}: max|d out|/max|V| = {err:.3e} (tol {tol:.0e}), max|d lse| = {lerr:.3e}")
    assert err <= tol, f"{what}: output error {err:.3e} > {tol:.0e}"
    assert lerr <= ltol, f"{what}: lse error {lerr:.3e} > {ltol:.0e}"
    return err, lerr


def check_full(case, n_splits=0, path=None, what="", fused_merge=None):
    out, lse, plan = run_gpu(case, n_splits, path, fused_merge=fused_merge, poison=True)
    if path in ("valu", "mfma"):
        assert plan["path"] == path
    ref_out, ref_lse = oracle_full(case)
    return compare(case, out, lse, ref_out, ref_lse, max_abs_v(case), what or case.spec.name), plan


def run_gpu_append(case, k_new, v_new, n_splits=0, path=None, fused_merge=None, poison=False):
    """fd_append_decode on the GPU; returns host (out, lse, k_after, v_after,
    plan).  case.k / case.v are updated in place."""
    dec = Decoder(case.q, case.k, case.v, scale=case.spec.scale, page_table=case.page_table,
                  seq_lens=case.seq_lens, T=case.spec.T if case.page_table is not None else None,
                  n_splits=n_splits, path=path, fused_merge=fused_merge, k_new=k_new, v_new=v_new)
    if poison and dec.workspace is not None:
        dec.workspace.fill_(0xFF)
    announce(f"append-decode {case.spec.name} B={case.spec.B} Hq={case.spec.Hq} Hkv={case.spec.Hkv} "
             f"T={case.spec.T} D={case.spec.D} {case.spec.dtype} seed={case.spec.seed} "
             f"n_splits={n_splits} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    return (out.cpu().double().numpy(), lse.cpu().double().numpy(), case.k.cpu(), case.v.cpu(),
            dec.plan)


def oracle_append(case_host, k_new_host, v_new_host):
    """The oracle's append-then-decode on host copies taken before the call."""
    c = case_host
    return oracle_mod.default().append_decode(c.q, k_new_host, v_new_host, c.k, c.v, c.spec.scale,
                                              c.seq_lens, page_table=c.page_table)


def check_append(case, k_new, v_new, n_splits=0, path=None, fused_merge=None, what=""):
    """Run fd_append_decode and compare out / lse with the oracle (tolerance
    as decode) and the caches after the call with the oracle's, bit for
    bit."""
    host = case.to("cpu")
    kn, vn = k_new.cpu(), v_new.cpu()
    ref_out, ref_lse, ref_k, ref_v = oracle_append(host, kn, vn)
    out, lse, k_after, v_after, plan = run_gpu_append(case, k_new, v_new, n_splits, path,
                                                      fused_merge, poison=True)
    if path in ("valu", "mfma"):
        assert plan["path"] == path
    # max |V| over the values attended to: the cached ones and the new rows
    vmax = max(max_abs_v(host), float(vn.abs().max()))
    err = compare(case, out, lse, ref_out, ref_lse, vmax, what or case.spec.name)
    raw = (lambda t: t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy())
    ka, va = raw(k_after), raw(v_after)
    rk = ref_k.view(np.int16) if ref_k.dtype == np.uint16 else ref_k
    rv = ref_v.view(np.int16) if ref_v.dtype == np.uint16 else ref_v
    assert np.array_equal(ka, rk) and np.array_equal(va, rv), f"{what}: caches after the append differ"
    return err, plan


def seq_host(case, b):
    """Host copies of sequence b of a case: (k, v, page_table, seq_lens) for
    the oracle.  A paged sequence gets its own pages, renumbered 0..n-1
    (same values, same order); a contiguous one its [1, Hkv, T, D] slice."""
    s = case.spec
    if case.page_table is None:
        sl = None if case.seq_lens is None else case.seq_lens[b:b + 1].cpu()
        return case.k[b:b + 1].cpu(), case.v[b:b + 1].cpu(), None, sl
    n = max(1, -(-case.lengths()[b] // s.page_size))
    pages = case.page_table[b, :n].long()
    table = torch.arange(n, dtype=torch.int32)[None]
    return case.k[pages].cpu(), case.v[pages].cpu(), table, case.seq_lens[b:b + 1].cpu()


def all_rows(case, out, lse, what=""):
    """Every (b, h) row of a large case against the oracle, one sequence at a
    time from host copies.  Each sequence's error is taken relative to its
    own max |V| (at most the whole case's).  Returns and reports the worst
    max|d out|/max|V| and max|d lse| over all rows."""
    s = case.spec
    orc = oracle_mod.default()
    worst = (0.0, 0.0)
    for b in range(s.B):
        k, v, table, sl = seq_host(case, b)
        ro, rl = orc.decode(case.q[b:b + 1].cpu(), k, v, s.scale, page_table=table, seq_lens=sl)
        vmax = max_abs_v(case, b)
        go, gl = out[b:b + 1], lse[b:b + 1]
        assert np.all(np.isfinite(go)), f"{what} b={b}: non-finite output"
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(gl)) and np.all(gl[~fin] == rl[~fin]), f"{what} b={b}: lse infinities"
        err = float(np.max(np.abs(go - ro))) / max(vmax, 1e-30)
        lerr = float(np.max(np.abs(gl[fin] - rl[fin]), initial=0.0))
        worst = (max(worst[0], err), max(worst[1], lerr))
    tol, ltol = OUT_TOL[s.dtype], LSE_TOL[s.dtype]
    announce(f"{what}: all {s.B * s.Hq} rows: max|d out|/max|V| = {worst[0]:.3e} (tol {tol:.0e}), "
             f"max|d lse| = {worst[1]:.3e} (tol {ltol:.0e})")
    assert worst[0] <= tol, f"{what}: output error {worst[0]:.3e} > {tol:.0e}"
    assert worst[1] <= ltol, f"{what}: lse error {worst[1]:.3e} > {ltol:.0e}"
    return worst


def all_queries(case, q, out, lse, bs, causal, what="", heads=None):
    """Every query of the sequences bs (all query heads, or the kv groups
    whose query heads are listed in `heads`) against the oracle's
    several-query decode of that sequence alone."""
    s = case.spec
    orc = oracle_mod.default()
    worst = (0.0, 0.0)
    for b in bs:
        k, v, table, sl = seq_host(case, b)
        qb = q[b:b + 1].cpu()
        hs = list(range(s.Hq)) if heads is None else list(heads)
        if heads is not None:
            # whole kv groups only: query heads j*G .. j*G+G-1 read kv head j
            kvh = sorted(set(h // s.G for h in hs))
            hs = [j * s.G + g for j in kvh for g in range(s.G)]
            qb = qb[:, :, hs].contiguous()
            # kv heads are axis 1 of a contiguous slice and of a page pool alike
            k, v = k[:, kvh].contiguous(), v[:, kvh].contiguous()
        ro, rl = orc.decode_multi(qb, k, v, s.scale, causal=causal, page_table=table, seq_lens=sl)
        go = out[b:b + 1][:, :, hs]
        gl = lse[b:b + 1][:, :, hs]
        vmax = max_abs_v(case, b)
        assert np.all(np.isfinite(go)), f"{what} b={b}: non-finite output"
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(gl)) and np.all(gl[~fin] == rl[~fin]), f"{what} b={b}: lse infinities"
        err = float(np.max(np.abs(go - ro))) / max(vmax, 1e-30)
        lerr = float(np.max(np.abs(gl[fin] - rl[fin]), initial=0.0))
        announce(f"{what} b={b}: {q.shape[1]} queries x {len(hs)} heads: err {err:.2e} lse {lerr:.2e}")
        worst = (max(worst[0], err), max(worst[1], lerr))
    tol, ltol = OUT_TOL[s.dtype], LSE_TOL[s.dtype]
    assert worst[0] <= tol, f"{what}: output error {worst[0]:.3e} > {tol:.0e}"
    assert worst[1] <= ltol, f"{what}: lse error {worst[1]:.3e} > {ltol:.0e}"
    return worst
