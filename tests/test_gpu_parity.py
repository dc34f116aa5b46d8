"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.  Small cases are compared element by element; the
full-size workloads, in the launch configuration the benchmark times, are
compared on sampled (batch, head) rows."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as oracle_mod
from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def small_case(name, device=DEV, **kw):
    return inputs.make_case(inputs.spec(name, **kw), device="cpu").to(device)


# ------------------------------------------------------------------ the five workloads, reduced

def test_tiny_f32_four_splits():
    case = small_case("tiny_f32")
    (err, _), plan = parity.check_full(case, n_splits=4)
    assert (plan["n_splits"], plan["chunk"]) == (4, 256)


@pytest.mark.parametrize("n", [0, 1, 8, 32, 128])
def test_mha_f16_split_sweep(n):
    case = small_case("mha32k_f16", Hq=8, Hkv=8, T=4096 + 37)
    parity.check_full(case, n_splits=n, what=f"mha f16 n={n}")


def test_gqa_bf16_spiky_keys():
    case = small_case("gqa128k_bf16", B=2, T=8192 + 5)
    parity.check_full(case, what="gqa bf16 spiky")


def test_paged_ragged_bf16():
    case = small_case("paged_ragged_bf16", B=5, T=3000, len_lo=1, len_hi=3000)
    for n in (0, 1, 7):
        parity.check_full(case, n_splits=n, what=f"paged n={n}")


def test_high_batch_gqa_hot_head():
    case = small_case("gqa_b64_bf16", B=4, T=2048 + 100)
    parity.check_full(case, what="b64 hot q")


# ------------------------------------------------------------------ shapes and group sizes

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_group_sizes(dtype, D, G, path):
    if path == "mfma" and dtype == "f32":
        pytest.skip("the matrix-core path takes f16 / bf16 inputs")
    Hkv = 2
    case = small_case("mha32k_f16", B=2, Hq=Hkv * G, Hkv=Hkv, D=D, T=700, dtype=dtype)
    parity.check_full(case, path=path, what=f"G={G} D={D} {dtype} {path}")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 257])
@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_short_sequences(T, path):
    case = small_case("gqa128k_bf16", B=1, Hq=8, Hkv=2, T=T)
    for n in (0, 1, 3):
        parity.check_full(case, n_splits=n, path=path, what=f"T={T} n={n} {path}")


@pytest.mark.parametrize("fused", [False, True])
def test_ragged_lengths_with_empty_sequences(fused):
    s = inputs.spec("mha32k_f16", B=4, Hq=4, Hkv=2, T=300)
    case = inputs.make_case(s).to(DEV)
    case.seq_lens = torch.tensor([0, 1, 299, 300], dtype=torch.int32, device=DEV)
    ref_out, ref_lse = parity.oracle_full(case)
    for n in (0, 1, 5):
        out, lse, plan = parity.run_gpu(case, n, fused_merge=fused, poison=True)
        if plan["n_splits"] > 1:
            assert plan["fused"] == fused
        parity.compare(case, out, lse, ref_out, ref_lse, parity.max_abs_v(case), f"ragged n={n}")
        assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_paged_page_sizes(path):
    for P in (1, 4, 16, 64, 256):
        case = small_case("paged_ragged_bf16", B=3, Hq=8, Hkv=4, T=1000, page_size=P,
                          len_lo=1, len_hi=1000)
        parity.check_full(case, path=path, what=f"page_size={P} {path}")


def test_paged_invalid_page_ids_read_as_empty():
    # Page ids outside [0, num_pages) are skipped instead of read; a table
    # whose second page is invalid equals the sequence cut after page one.
    s = inputs.spec("paged_ragged_bf16", B=1, Hq=8, Hkv=2, T=64, len_lo=64, len_hi=64)
    case = inputs.make_case(s).to(DEV)
    bad = case.page_table.clone()
    bad[0, 1:] = case.k.shape[0] + 5
    cut = inputs.Case(s, case.q, case.k, case.v, case.page_table,
                      torch.tensor([16], dtype=torch.int32, device=DEV))
    for path in ("valu", "mfma"):
        a = parity.run_gpu(inputs.Case(s, case.q, case.k, case.v, bad, case.seq_lens), 1, path)
        b = parity.run_gpu(cut, 1, path)
        assert np.max(np.abs(a[0] - b[0])) <= 1e-6 and np.max(np.abs(a[1] - b[1])) <= 1e-6


def test_paged_equals_contiguous_gather():
    s = inputs.spec("paged_ragged_bf16", B=3, T=900, len_lo=600, len_hi=900)
    case = inputs.make_case(s).to(DEV)
    out_p, lse_p, _ = parity.run_gpu(case, 4)
    lens = case.lengths()
    k = torch.zeros((s.B, s.Hkv, s.T, s.D), dtype=case.k.dtype, device=DEV)
    v = torch.zeros_like(k)
    for b in range(s.B):
        t = torch.arange(lens[b], device=DEV)
        pages = case.page_table[b, t // s.page_size].long()
        k[b, :, :lens[b]] = case.k[pages, :, t % s.page_size].transpose(0, 1)
        v[b, :, :lens[b]] = case.v[pages, :, t % s.page_size].transpose(0, 1)
    cont = inputs.Case(s, case.q, k, v, None, case.seq_lens)
    out_c, lse_c, _ = parity.run_gpu(cont, 4)
    assert np.max(np.abs(out_p - out_c)) <= 1e-6 and np.max(np.abs(lse_p - lse_c)) <= 1e-6


# ------------------------------------------------------------------ closed-form cases on the GPU

def test_special_values_on_gpu():
    s = inputs.spec("gqa128k_bf16", B=1, Hq=8, Hkv=2, T=1000)
    case = inputs.make_case(s).to(DEV)
    # constant V -> that constant
    v = torch.empty_like(case.v)
    v[:] = case.v[:, :, :1]
    c = inputs.Case(s, case.q, case.k, v)
    out, _, _ = parity.run_gpu(c, 4)
    ref = case.v[:, :, 0].float().repeat_interleave(4, dim=1).cpu().numpy()
    assert np.max(np.abs(out - ref)) <= 1e-6 * max(1.0, np.abs(ref).max())
    # q = 0 -> mean of V, lse = ln T
    c = inputs.Case(s, torch.zeros_like(case.q), case.k, case.v)
    out, lse, _ = parity.run_gpu(c, 4)
    mean = case.v.double().mean(dim=2).repeat_interleave(4, dim=1).cpu().numpy()
    assert np.max(np.abs(out - mean)) <= 1e-5
    assert np.max(np.abs(lse - math.log(1000))) <= 1e-5


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_deterministic_runs(path):
    case = small_case("gqa128k_bf16", B=2, T=5000)
    a = parity.run_gpu(case, 0, path)
    b = parity.run_gpu(case, 0, path)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_fused_merge_with_stale_workspace(path):
    # The arrival counters carry a per-call tag: a workspace full of garbage
    # (NaN partials, foreign tags) before every call, or left by a call with
    # another split count or other inputs, must not change results.  Inputs
    # alternate so a stale partial could not pass for a fresh one.
    cases = [small_case("gqa128k_bf16", B=3, T=6000),
             small_case("gqa128k_bf16", B=3, T=6000, seed=301)]
    refs = [parity.oracle_full(c) for c in cases]
    vmax = [parity.max_abs_v(c) for c in cases]
    decs = {}
    for rep in range(4):
        for n in (7, 20):
            for i, c in enumerate(cases):
                key = (n, i)
                if key not in decs:
                    decs[key] = Decoder(c.q, c.k, c.v, scale=c.spec.scale, n_splits=n, path=path,
                                        fused_merge=True)
                dec = decs[key]
                assert dec.plan["fused"]
                if rep % 2 == 0:
                    dec.workspace.fill_(0xFF)
                parity.announce(f"fused merge n={n} case={i} rep={rep} {path}")
                out, lse = dec()
                torch.cuda.synchronize()
                parity.compare(c, out.cpu().double().numpy(), lse.cpu().double().numpy(),
                               refs[i][0], refs[i][1], vmax[i], f"fused n={n} case={i} rep={rep}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_fused_merge_matches_combine_kernel(path):
    # Many groups and splits finishing in arbitrary order: the fused merge
    # must agree with the separate combine kernel on every run.
    case = small_case("mha32k_f16", B=2, Hq=32, Hkv=8, T=20000)
    base = Decoder(case.q, case.k, case.v, scale=case.spec.scale, n_splits=40, path=path,
                   fused_merge=False)
    fused = Decoder(case.q, case.k, case.v, scale=case.spec.scale, n_splits=40, path=path,
                    fused_merge=True)
    assert not base.plan["fused"] and fused.plan["fused"]
    ref_out, ref_lse = (x.clone() for x in base())
    torch.cuda.synchronize()
    for rep in range(20):
        if rep % 3 == 0:       # garbage counters: the exchange-loop count; else one add each
            fused.workspace.fill_(0xFF)
        out, lse = fused()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"rep {rep}: non-finite output"
        assert torch.allclose(out, ref_out, rtol=0, atol=2e-6) and torch.allclose(lse, ref_lse, rtol=0, atol=2e-6), f"rep {rep}"


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_fused_merge_ragged_and_paged(path):
    case = small_case("paged_ragged_bf16", B=6, T=5000, len_lo=0, len_hi=5000)
    case.seq_lens[1] = 0
    for n in (0, 3, 11):
        parity.check_full(case, n_splits=n, path=path, fused_merge=True, what=f"fused paged n={n}")


# ------------------------------------------------------------------ balanced stream mode (paged, automatic plans)

@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("wgs", [1, 3, 8, 64, 1000])
def test_stream_mode_workgroup_counts(monkeypatch, path, wgs):
    # Rows laid end to end and cut into `wgs` equal ranges: one workgroup
    # covering everything, rows split over several workgroups, rows shorter
    # than a range, and more workgroups than tiles.  Empty sequences and a
    # poisoned workspace included.
    monkeypatch.setenv("FD_STREAM_WGS", str(wgs))
    for P in (16, 256):
        case = small_case("paged_ragged_bf16", B=7, Hq=8, Hkv=2, T=5000, page_size=P,
                          len_lo=0, len_hi=5000)
        case.seq_lens[2] = 0
        case.seq_lens[4] = 1
        (_, _), plan = parity.check_full(case, path=path, what=f"stream wgs={wgs} P={P} {path}")
        assert plan["stream"] and plan["n_splits"] == wgs


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("row_cost", [0, 64, 1000, 20000])
def test_stream_mode_row_cost(monkeypatch, path, row_cost):
    # Positions before each row's tokens move the range boundaries: ranges
    # that end before a row's first token (an empty segment), rows shorter
    # than the positions before them, and a cost longer than any range.
    monkeypatch.setenv("FD_STREAM_WGS", "13")
    monkeypatch.setenv("FD_STREAM_ROWCOST", str(row_cost))
    case = small_case("paged_ragged_bf16", B=9, Hq=8, Hkv=2, T=3000, page_size=16, len_lo=0, len_hi=3000)
    case.seq_lens[1] = 0
    case.seq_lens[3] = 1
    case.seq_lens[5] = 129
    (_, _), plan = parity.check_full(case, path=path, what=f"stream row cost {row_cost} {path}")
    assert plan["stream"] and plan["n_splits"] == 13


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_stream_mode_merge_cap(monkeypatch, path):
    # Many workgroups over one long row: ranges are widened so that no row
    # is cut into more pieces than the in-launch merge holds.
    monkeypatch.setenv("FD_STREAM_WGS", "1000")
    case = small_case("paged_ragged_bf16", B=2, Hq=32, Hkv=1, T=40000, len_lo=30000, len_hi=40000)
    (_, _), plan = parity.check_full(case, path=path, what=f"stream merge cap {path}")
    assert plan["stream"]


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_stream_mode_long_ranges_restage_pages(monkeypatch, path):
    # A range longer than the on-chip page-id stage (2048 pages), starting
    # inside a page: 256-token pages, ranges cut at multiples of the tile.
    # Two workgroups: each range spans a little over 2048 pages and the
    # second one starts three quarters into a page.
    monkeypatch.setenv("FD_STREAM_WGS", "2")
    T = 2 * (2048 * 256 + 128 * 3) + 50
    case = small_case("paged_ragged_bf16", B=1, Hq=4, Hkv=1, D=64, T=T, page_size=256,
                      len_lo=T, len_hi=T)
    (_, _), plan = parity.check_full(case, path=path, what=f"stream restage {path}")
    assert plan["stream"]


def test_fused_plans_sharing_one_workspace():
    # A stream plan and a split-grid plan with other row counts take turns
    # on one workspace: each call must count its arrivals correctly from the
    # counters the other plan left (tagged for another call, or untouched).
    case = small_case("paged_ragged_bf16", B=6, Hq=8, Hkv=2, T=4000, len_lo=0, len_hi=4000)
    case.seq_lens[3] = 0
    other = small_case("mha32k_f16", B=3, Hq=16, Hkv=4, T=3000, dtype="bf16")
    decs = [Decoder(case.q, case.k, case.v, scale=case.spec.scale, page_table=case.page_table,
                    seq_lens=case.seq_lens, T=case.spec.T),
            Decoder(case.q, case.k, case.v, scale=case.spec.scale, page_table=case.page_table,
                    seq_lens=case.seq_lens, T=case.spec.T, n_splits=7, fused_merge=True),
            Decoder(other.q, other.k, other.v, scale=other.spec.scale, n_splits=9, fused_merge=True)]
    assert decs[0].plan["stream"] and decs[1].plan["fused"] and decs[2].plan["fused"]
    size = max(d.plan["workspace_bytes"] for d in decs)
    shared = torch.empty(size, dtype=torch.uint8, device=DEV)
    shared.fill_(0xFF)
    for d in decs:
        d.opt.workspace = shared.data_ptr()
        d.opt.workspace_bytes = size
    cases = [case, case, other]
    refs = [parity.oracle_full(c) for c in cases]
    vmax = [parity.max_abs_v(c) for c in cases]
    for rep, i in enumerate([0, 1, 0, 0, 2, 1, 1, 2, 0, 2, 2, 1]):
        parity.announce(f"shared workspace rep={rep} plan={i}")
        out, lse = decs[i]()
        torch.cuda.synchronize()
        parity.compare(cases[i], out.cpu().double().numpy(), lse.cpu().double().numpy(),
                       refs[i][0], refs[i][1], vmax[i], f"shared workspace rep={rep} plan={i}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_split_and_combine_entry_points(path):
    case = small_case("gqa128k_bf16", B=2, Hq=8, Hkv=2, T=3000)
    ref_out, ref_lse = parity.oracle_full(case)
    vmax = parity.max_abs_v(case)
    for n in (6, 100):
        dec = Decoder(case.q, case.k, case.v, scale=case.spec.scale, n_splits=n, path=path,
                      fused_merge=True)
        assert dec.plan["n_splits"] > 1
        parity.announce(f"fd_split + fd_combine separately n={n} {path}")
        dec.split()
        dec.combine()
        torch.cuda.synchronize()
        out1, lse1 = dec.out.cpu().double().numpy(), dec.lse.cpu().double().numpy()
        parity.compare(case, out1, lse1, ref_out, ref_lse, vmax, f"separate passes n={n}")
        dec()
        torch.cuda.synchronize()
        out2, lse2 = dec.out.cpu().double().numpy(), dec.lse.cpu().double().numpy()
        parity.compare(case, out2, lse2, ref_out, ref_lse, vmax, f"fd_decode n={n}")
        assert np.max(np.abs(out1 - out2)) <= 1e-6 and np.max(np.abs(lse1 - lse2)) <= 1e-6


# ------------------------------------------------------------------ full-size workloads, every row

def test_full_mha32k_f16_split_sweep():
    s = inputs.spec("mha32k_f16")
    case = inputs.make_case(s, device=DEV)
    for n in (0, 1, 8, 32, 128):
        out, lse, plan = parity.run_gpu(case, n)
        parity.all_rows(case, out, lse, f"mha32k n={n} ({plan['n_splits']} splits)")


def test_full_gqa128k_bf16():
    s = inputs.spec("gqa128k_bf16")
    case = inputs.make_case(s, device=DEV)
    out, lse, _ = parity.run_gpu(case, 0)
    parity.all_rows(case, out, lse, "gqa128k")


def test_full_paged_ragged_bf16():
    s = inputs.spec("paged_ragged_bf16")
    case = inputs.make_case(s, device=DEV)
    out, lse, plan = parity.run_gpu(case, 0)
    assert plan["stream"]
    lens = case.lengths()
    assert any(n % s.page_size for n in lens)
    parity.all_rows(case, out, lse, "paged ragged")


def test_full_gqa_b64_bf16_hot_heads():
    s = inputs.spec("gqa_b64_bf16")
    case = inputs.make_case(s, device=DEV)
    out, lse, _ = parity.run_gpu(case, 0)
    parity.all_rows(case, out, lse, "b64 gqa")
    del out, lse, case
    torch.cuda.empty_cache()


def test_largest_contiguous_slice():
    # one (batch, kv head) slice just under 4 GiB -- the largest the kernels'
    # 32-bit offsets address (2^24 - 32 tokens x 128 x 2 bytes) -- through
    # the vector and matrix-core split kernels and, with 8 causal queries
    # (32 rows per kv head), the split kernel's two row blocks and the
    # query-tiled kernel with its KV splits;
    # sampled against the oracle
    T = (1 << 24) - 32
    s = inputs.spec("gqa128k_bf16", B=1, Hq=4, Hkv=1, T=T)
    case = inputs.make_case(s, device=DEV)
    parity.announce(f"largest slice T={T}: host copies for the oracle")
    k_h, v_h = case.k.cpu(), case.v.cpu()
    vmax = float(v_h.abs().max())
    orc = oracle_mod.default()
    ref, ref_l = orc.decode(case.q.cpu(), k_h, v_h, s.scale)
    for path in ("valu", "mfma"):
        out, lse, plan = parity.run_gpu(case, 0, path=path)
        assert plan["path"] == path
        err = float(np.max(np.abs(out - ref))) / vmax
        lerr = float(np.max(np.abs(lse - ref_l)))
        parity.announce(f"largest slice {path}: err {err:.2e} lse {lerr:.2e}")
        assert err <= parity.OUT_TOL["bf16"] and lerr <= parity.LSE_TOL["bf16"]
    nq = 8
    q = inputs.make_q_multi(s, nq, device=DEV)
    refs = {i: orc.decode(q[:, i].cpu(), k_h, v_h, s.scale, seq_lens=np.array([T - (nq - 1 - i)], np.int32))
            for i in (0, nq - 1)}
    # 32 rows per kv head: the automatic plan takes the split kernel's two
    # row blocks; the query-tiled kernel with its KV splits is asked for
    for path, want in ((None, "mfma"), ("prefill", "prefill")):
        dec = Decoder(q, case.k, case.v, scale=s.scale, causal=True, path=path)
        assert dec.plan["path"] == want and dec.plan["n_splits"] > 1
        parity.announce(f"largest slice {want} plan={dec.plan}")
        out, lse = dec()
        torch.cuda.synchronize()
        for i, (r, rl) in refs.items():
            err = float(np.max(np.abs(out[0, i].cpu().double().numpy() - r[0]))) / vmax
            lerr = float(np.max(np.abs(lse[0, i].cpu().double().numpy() - rl[0])))
            parity.announce(f"largest slice {want} query={i}: err {err:.2e} lse {lerr:.2e}")
            assert err <= parity.OUT_TOL["bf16"] and lerr <= parity.LSE_TOL["bf16"]
        del dec, out, lse
    del q, case, k_h, v_h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,layout", [(2048, "paged"), (2049, "paged"), (65535, "contiguous")])
def test_many_sequences(B, layout):
    # batch-size edges: stream mode scans at most 2048 sequences on chip
    # (one more falls back to the split grid), and B = 65535 is the largest
    # grid the split kernels take; short ragged sequences, some empty
    if layout == "paged":
        s = inputs.spec("paged_ragged_bf16", B=B, Hq=8, Hkv=2, D=64, T=48, page_size=16, len_lo=0, len_hi=48)
    else:
        s = inputs.spec("gqa128k_bf16", B=B, Hq=4, Hkv=1, D=64, T=8)
    case = inputs.make_case(s).to(DEV)
    (_, _), plan = parity.check_full(case, what=f"B={B} {layout}")
    if layout == "paged":
        assert plan["stream"] == (B <= 2048)


def test_many_sequences_query_tiled():
    # the query-tiled kernel's grid at a large batch (z = B), with KV splits
    s = inputs.spec("gqa128k_bf16", B=3000, Hq=4, Hkv=1, D=64, T=40)
    case = inputs.make_case(s).to(DEV)
    from tests.test_gpu_multi import check_multi
    q = inputs.make_q_multi(s, 20).to(DEV)
    for n in (0, 2):
        plan = check_multi(case, q, True, n_splits=n, what=f"query-tiled B=3000 n={n}")
        assert plan["path"] == "prefill"
