"""fd_decode_noalloc through the C ABI: the same results as fd_decode with a
caller-owned workspace (bit for bit: same plan, same kernels) and within the
oracle's tolerance, on calls in a row where each following call is smaller
than the one before, so the static scratch holds a larger call's partials
and counters when a smaller one starts.  Contiguous and paged (stream mode)
plans, in-launch merge and combine kernel, and ragged paged query-tiled calls
whose column order and split size the order pass writes into the scratch."""
import numpy as np
import pytest
import torch

from split_kv_fd_amd import fd, inputs
from split_kv_fd_amd.decode import Decoder, FDError, make_options
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(name, **kw):
    return inputs.make_case(inputs.spec(name, **kw), device="cpu")


def _noalloc(case_dev, spec, fused_merge=None):
    """One fd_decode_noalloc call; returns (out, lse) on the host."""
    q, k, v = case_dev.q, case_dev.k, case_dev.v
    paged = case_dev.page_table is not None
    B, Hq, D = q.shape[0], q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    T = spec.T
    opt = make_options(q.dtype, page_size=k.shape[2] if paged else 0,
                       max_pages=case_dev.page_table.shape[1] if paged else 0,
                       num_pages=k.shape[0] if paged else 0, fused_merge=fused_merge)
    opt.stream = torch.cuda.current_stream().cuda_stream
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = fd.fd_decode_noalloc(ptr(q), ptr(k), ptr(v), ptr(case_dev.page_table), ptr(case_dev.seq_lens),
                              out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, T, D, spec.scale, 0, opt)
    if st != fd.FD_OK:
        raise FDError(st, "fd_decode_noalloc")
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def _check(case, fused_merge=None, what=""):
    s = case.spec
    dev = case.to(DEV)
    dec = Decoder(dev.q, dev.k, dev.v, scale=s.scale, page_table=dev.page_table, seq_lens=dev.seq_lens,
                  T=s.T if dev.page_table is not None else None, fused_merge=fused_merge)
    assert dec.plan["workspace_bytes"] <= fd.FD_NOALLOC_SCRATCH_BYTES
    parity.announce(f"noalloc {what}: {s.name} B={s.B} Hq={s.Hq} Hkv={s.Hkv} T={s.T} plan={dec.plan}")
    out, lse = _noalloc(dev, s, fused_merge)
    ref_gpu = dec()
    torch.cuda.synchronize()
    ref_out, ref_lse = (x.cpu().double().numpy() for x in ref_gpu)
    assert np.array_equal(out, ref_out), f"{what}: out differs from fd_decode"
    assert np.array_equal(lse, ref_lse), f"{what}: lse differs from fd_decode"
    o_out, o_lse = parity.oracle_full(case)
    parity.compare(case, out, lse, o_out, o_lse, parity.max_abs_v(case), f"noalloc {what}")
    return dec.plan


def test_noalloc_matches_fd_decode_larger_then_smaller():
    big = _case("gqa128k_bf16", B=3, T=20000)
    small = _case("mha32k_f16", Hq=8, Hkv=8, T=3000)
    p1 = _check(big, what="call 1 (larger)")
    p2 = _check(small, what="call 2 (smaller)")
    assert p1["n_splits"] > 1 and p2["n_splits"] > 1
    assert p1["workspace_bytes"] > p2["workspace_bytes"]


def test_noalloc_paged_stream_then_smaller_and_combine_kernel():
    big = _case("paged_ragged_bf16", B=8, Hq=16, Hkv=4, T=12000, len_lo=0, len_hi=12000)
    big.seq_lens[1] = 0
    small = _case("paged_ragged_bf16", B=3, Hq=8, Hkv=2, T=5000, len_lo=100, len_hi=5000)
    p1 = _check(big, what="paged call 1 (larger, stream mode)")
    p2 = _check(small, what="paged call 2 (smaller, stream mode)")
    assert p1["stream"] and p2["stream"]
    assert p1["workspace_bytes"] > p2["workspace_bytes"]
    # a plan whose splits the combine kernel merges, then a smaller fused one
    mid = _case("gqa128k_bf16", B=2, T=9000)
    p3 = _check(mid, fused_merge=False, what="call 3 (combine kernel)")
    p4 = _check(small, what="call 4 (smaller, stream mode again)")
    assert not p3["fused"] and p3["n_splits"] > 1 and p4["stream"]


def _noalloc_multi(case_dev, spec, q, causal):
    """fd_decode_noalloc with several queries per sequence; (out, lse) on the host."""
    k, v = case_dev.k, case_dev.v
    B, nq, Hq, D = q.shape
    opt = make_options(q.dtype, page_size=k.shape[2], max_pages=case_dev.page_table.shape[1],
                       num_pages=k.shape[0], n_queries=nq, causal=causal)
    opt.stream = torch.cuda.current_stream().cuda_stream
    out = torch.full((B, nq, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, nq, Hq), float("nan"), dtype=torch.float32, device=DEV)
    st = fd.fd_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), case_dev.page_table.data_ptr(),
                              case_dev.seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, k.shape[1],
                              spec.T, D, spec.scale, 0, opt)
    if st != fd.FD_OK:
        raise FDError(st, "fd_decode_noalloc")
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def test_noalloc_query_tiled_ordered_then_smaller():
    # ragged paged calls with 16 causal queries: the order pass's column
    # order and the split size it picks live in the static scratch too; a
    # larger call, then a smaller one, each bit for bit fd_decode's result
    # and within the oracle's tolerance
    from oracle import oracle as oracle_mod
    for i, (B, T) in enumerate(((6, 9000), (3, 4000))):
        s = inputs.spec("paged_ragged_bf16", B=B, Hq=8, Hkv=2, T=T, len_lo=0, len_hi=T)
        case = inputs.make_case(s, device="cpu")
        case.seq_lens[min(1, B - 1)] = 0
        dev = case.to(DEV)
        q = inputs.make_q_multi(s, 16).to(DEV)
        dec = Decoder(q, dev.k, dev.v, scale=s.scale, page_table=dev.page_table, seq_lens=dev.seq_lens, T=T,
                      causal=True)
        assert dec.plan["path"] == "prefill" and dec.plan["head_blocks"] == 1 and dec.plan["n_splits"] > 1
        assert dec.plan["workspace_bytes"] <= fd.FD_NOALLOC_SCRATCH_BYTES
        parity.announce(f"noalloc query-tiled call {i + 1}: B={B} T={T} plan={dec.plan}")
        out, lse = _noalloc_multi(dev, s, q, True)
        ref_gpu = dec()
        torch.cuda.synchronize()
        ref_out, ref_lse = (x.cpu().double().numpy() for x in ref_gpu)
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), f"call {i + 1}: differs from fd_decode"
        o_out, o_lse = oracle_mod.default().decode_multi(q.cpu(), case.k, case.v, s.scale, causal=True,
                                                         page_table=case.page_table, seq_lens=case.seq_lens)
        parity.compare(case, out, lse, o_out, o_lse, parity.max_abs_v(case), f"noalloc query-tiled call {i + 1}")
