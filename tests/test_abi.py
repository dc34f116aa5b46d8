"""The C ABI on the host (no GPU work): symbols, defaults, the planner and
argument checking.  Every call here either fails validation before any
launch or is a host-only planning call."""
import ctypes
import os
import re

import pytest
import torch

from split_kv_fd_amd import fd
from split_kv_fd_amd.inputs import SPECS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fd.LIB_PATH):
        from split_kv_fd_amd import build
        build.build()
    return fd.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert declared == sorted(fd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_struct_sizes_match_header(lib):
    # fd_options_init writes struct_size = sizeof(fd_options_t) of the library.
    opt = fd.fd_options_t()
    fd.fd_options_init(opt)
    assert opt.struct_size == ctypes.sizeof(fd.fd_options_t)
    assert opt.dtype == fd.FD_BF16 and opt.path == fd.FD_PATH_AUTO
    assert opt.workspace is None and opt.stream is None and opt.page_size == 0
    assert opt.n_queries == 1 and opt.causal == 0


def opts(dtype=fd.FD_BF16, **kw):
    o = fd.fd_options_t()
    fd.fd_options_init(o)
    o.dtype = dtype
    o.num_cus = kw.pop("num_cus", 256)
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def plan(B, Hq, Hkv, T, D, n=0, **kw):
    p = fd.fd_plan_t()
    st = fd.fd_plan(B, Hq, Hkv, T, D, n, opts(**kw), p)
    return st, p


def test_plan_covers_sequence_and_respects_tiles(lib):
    for (B, Hq, Hkv, T, D) in [(1, 32, 32, 32768, 128), (4, 32, 8, 131072, 128),
                               (64, 64, 8, 32768, 128), (1, 4, 4, 1024, 64), (3, 6, 2, 1000, 64),
                               (1, 1, 1, 1, 128)]:
        for n in (0, 1, 3, 8, 32, 128, 100000):
            for dt in (fd.FD_F32, fd.FD_F16, fd.FD_BF16):
                st, p = plan(B, Hq, Hkv, T, D, n, dtype=dt)
                assert st == fd.FD_OK, fd.fd_last_error()
                assert p.n_splits >= 1 and p.chunk % 16 == 0
                assert p.chunk * p.n_splits >= T > p.chunk * (p.n_splits - 1)
                if n:
                    assert p.n_splits <= n
                assert p.grid[0] == p.n_splits and p.grid[2] == B
                assert p.grid[1] == Hkv * p.head_blocks
                assert p.heads_per_block * p.head_blocks >= Hq // Hkv
                assert bool(p.combine) == (p.n_splits > 1)
                assert not p.fused or (p.combine and p.n_splits * min(Hq // Hkv, p.heads_per_block) <= 1024)
                assert not p.fused or B * Hkv * p.head_blocks * p.n_splits <= 512
                parts = B * Hq * p.n_splits
                if p.n_splits > 1:
                    assert p.workspace_bytes >= parts * (D + 2) * 4 + B * Hkv * p.head_blocks * 8
                else:
                    assert p.workspace_bytes == 0
                G = Hq // Hkv
                want_mfma = dt != fd.FD_F32 and G >= 4   # contiguous caches
                assert p.path == (fd.FD_PATH_MFMA if want_mfma else fd.FD_PATH_VALU)
                assert p.heads_per_block == (16 if want_mfma else min(8, 1 << (G - 1).bit_length()))


def test_plan_of_the_five_workloads(lib):
    # The tiny fp32 case asks for 4 splits of 256 tokens.
    st, p = plan(1, 4, 4, 1024, 64, 4, dtype=fd.FD_F32)
    assert st == fd.FD_OK and (p.n_splits, p.chunk) == (4, 256)
    # Automatic plans put at least one workgroup on every compute unit when
    # the sequence allows it, and give high-batch GQA a single split.
    for name in ("mha32k_f16", "gqa128k_bf16", "gqa_b64_bf16"):
        s = SPECS[name]
        dt = {"f16": fd.FD_F16, "bf16": fd.FD_BF16}[s.dtype]
        st, p = plan(s.B, s.Hq, s.Hkv, s.T, s.D, 0, dtype=dt)
        assert st == fd.FD_OK
        assert p.grid[0] * p.grid[1] * p.grid[2] >= 256
    s = SPECS["gqa_b64_bf16"]
    st, p = plan(s.B, s.Hq, s.Hkv, s.T, s.D, 0)
    assert p.n_splits == 1


def test_plan_paged_chunks_align_to_pages(lib):
    # explicit split counts keep the split grid: chunks are whole pages
    st, p = plan(16, 32, 8, 65536, 128, 40, page_size=256, max_pages_per_seq=256, num_pages=10)
    assert st == fd.FD_OK and p.chunk % 256 == 0 and not p.stream
    assert p.chunk * p.n_splits >= 65536 and p.chunk <= 2048 * 256
    # a split stages at most 2048 page ids on chip
    st, p = plan(1, 8, 8, 65536, 128, 1, page_size=16, max_pages_per_seq=4096, num_pages=10)
    assert st == fd.FD_OK and p.chunk <= 2048 * 16 and p.n_splits >= 2
    assert plan(1, 4, 4, 100, 128, flags=8)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, flags=3)[0] == fd.FD_ERR_INVALID_ARG


@pytest.mark.parametrize("G,dtype,path", [(4, fd.FD_BF16, fd.FD_PATH_AUTO), (1, fd.FD_F16, fd.FD_PATH_AUTO),
                                          (8, fd.FD_F32, fd.FD_PATH_AUTO), (16, fd.FD_BF16, fd.FD_PATH_AUTO),
                                          (32, fd.FD_BF16, fd.FD_PATH_MFMA)])
def test_plan_paged_stream_mode(lib, G, dtype, path):
    # automatic plans of paged (ragged) batches on the split kernels use the
    # balanced stream mode: one workgroup per stream range and compute unit,
    # merged in-launch (32 query rows per kv head would take the query-tiled
    # kernel unless the matrix-core path is asked for)
    B, Hkv, D = 16, 2, 128
    st, p = plan(B, G * Hkv, Hkv, 65536, D, 0, dtype=dtype, page_size=16,
                 max_pages_per_seq=4096, num_pages=10, num_cus=100, path=path)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.stream and p.fused and p.combine and p.chunk == 0
    assert (p.n_splits, p.grid[0], p.grid[1], p.grid[2]) == (100, 100, 1, 1)
    assert p.block == 256
    rows = B * Hkv * p.head_blocks
    slots = (rows + p.n_splits) * p.heads_per_block
    assert p.workspace_bytes >= rows * 8 + slots * (D + 2) * 4
    assert p.tile > 0 and p.tile % 16 == 0
    # too many sequences for the on-chip prefix scan: the split grid
    st, p = plan(4096, G * Hkv, Hkv, 1024, D, 0, dtype=dtype, page_size=16,
                 max_pages_per_seq=64, num_pages=10, path=path)
    assert st == fd.FD_OK and not p.stream and p.chunk > 0


def test_plan_merge_choice(lib):
    # a small call in one round of workgroups: fused merge; many rounds, or
    # more than 48 MiB of K/V: combine kernel; the flags override either way
    st, p = plan(1, 32, 32, 2048, 128, 0, dtype=fd.FD_F16)          # 32 MiB of K/V
    assert st == fd.FD_OK and p.n_splits > 1 and p.fused
    st, p = plan(1, 32, 32, 3072, 128, 0, dtype=fd.FD_F16)          # 48 MiB
    assert st == fd.FD_OK and p.n_splits > 1 and p.fused
    st, p = plan(1, 32, 32, 3200, 128, 0, dtype=fd.FD_F16)          # just over
    assert st == fd.FD_OK and p.n_splits > 1 and not p.fused
    st, p = plan(1, 32, 32, 32768, 128, 0, dtype=fd.FD_F16)         # 512 MiB
    assert st == fd.FD_OK and p.n_splits > 1 and not p.fused
    st, p = plan(1, 32, 32, 2048, 128, 64, dtype=fd.FD_F16)         # many rounds
    assert st == fd.FD_OK and not p.fused
    st, p = plan(1, 32, 32, 32768, 128, 64, dtype=fd.FD_F16, flags=fd.FD_FLAG_FUSED_MERGE)
    assert st == fd.FD_OK and p.fused
    st, p = plan(1, 32, 32, 2048, 128, 0, dtype=fd.FD_F16, flags=fd.FD_FLAG_COMBINE_KERNEL)
    assert st == fd.FD_OK and not p.fused


def test_plan_paths(lib):
    assert plan(1, 32, 8, 4096, 128, 0, path=fd.FD_PATH_MFMA, dtype=fd.FD_F32)[0] == fd.FD_ERR_UNSUPPORTED
    st, p = plan(1, 8, 8, 4096, 128, 0, path=fd.FD_PATH_MFMA, dtype=fd.FD_F16)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_MFMA and p.heads_per_block == 16
    # G = 32: one workgroup takes both 16-row blocks on a single K / V read
    st, p = plan(1, 64, 2, 4096, 128, 0, path=fd.FD_PATH_MFMA)
    assert st == fd.FD_OK and p.heads_per_block == 32 and p.head_blocks == 1 and p.grid[1] == 2
    st, p = plan(1, 128, 2, 4096, 128, 0, path=fd.FD_PATH_MFMA)  # G = 64: two 32-row blocks
    assert st == fd.FD_OK and p.heads_per_block == 32 and p.head_blocks == 2 and p.grid[1] == 4
    st, p = plan(1, 64, 8, 4096, 64, 0, path=fd.FD_PATH_VALU)     # G = 8 on the VALU path
    assert st == fd.FD_OK and p.path == fd.FD_PATH_VALU and p.heads_per_block == 8


def test_workspace_bytes_matches_plan(lib):
    o = opts(dtype=fd.FD_F16)
    p = fd.fd_plan_t()
    assert fd.fd_plan(1, 32, 32, 32768, 128, 16, o, p) == fd.FD_OK
    assert fd.fd_workspace_bytes(1, 32, 32, 32768, 128, 16, o) == p.workspace_bytes > 0
    assert fd.fd_workspace_bytes(1, 32, 32, 32768, 128, 1, o) == 0
    assert fd.fd_workspace_bytes(1, 3, 2, 32768, 128, 16, o) == 0   # invalid -> 0


@pytest.mark.parametrize("args,status", [
    ((1, 3, 2, 100, 128), fd.FD_ERR_INVALID_ARG),     # Hq % Hkv
    ((0, 4, 4, 100, 128), fd.FD_ERR_INVALID_ARG),
    ((1, 4, 4, 0, 128), fd.FD_ERR_INVALID_ARG),
    ((1, 4, 4, 100, -1), fd.FD_ERR_INVALID_ARG),
    ((1, 4, 4, 100, 96), fd.FD_ERR_UNSUPPORTED),
    ((1, 4, 4, 100, 256), fd.FD_ERR_UNSUPPORTED),
    ((1, 4, 4, 1 << 30, 128), fd.FD_ERR_UNSUPPORTED),  # 256 GiB per slice
])
def test_plan_rejects(lib, args, status):
    st, _ = plan(*args)
    assert st == status
    assert fd.fd_last_error() != ""


def test_plan_rejects_bad_options(lib):
    assert plan(1, 4, 4, 100, 128, -1)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, dtype=7)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, path=5)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, page_size=12, max_pages_per_seq=9, num_pages=1)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, page_size=16, max_pages_per_seq=6, num_pages=1)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, page_size=16, max_pages_per_seq=7, num_pages=0)[0] == fd.FD_ERR_INVALID_ARG
    o = opts()
    o.struct_size = 8
    p = fd.fd_plan_t()
    assert fd.fd_plan(1, 4, 4, 100, 128, 0, o, p) == fd.FD_ERR_INVALID_ARG
    lib_ = fd.load()
    assert lib_.fd_plan(1, 4, 4, 100, 128, 0, None, ctypes.byref(p)) == fd.FD_ERR_INVALID_ARG
    assert lib_.fd_plan(1, 4, 4, 100, 128, 0, ctypes.byref(o), None) == fd.FD_ERR_INVALID_ARG


# Pointer values below are never dereferenced: each call fails host
# validation before anything is launched.
A = 1 << 20          # 16-byte aligned fake address
MIS = A + 2          # misaligned


def decode(q=A, k=A, v=A, pt=None, sl=None, out=A, lse=A, shape=(1, 4, 4, 4096, 128), scale=0.1,
           n=16, **kw):
    return fd.fd_decode(q, k, v, pt, sl, out, lse, *shape, scale, n, opts(**kw))


def test_decode_rejects_before_launch(lib):
    assert decode(q=None) == fd.FD_ERR_INVALID_ARG
    assert decode(v=None) == fd.FD_ERR_INVALID_ARG
    assert decode(out=None) == fd.FD_ERR_INVALID_ARG
    assert decode(k=MIS) == fd.FD_ERR_INVALID_ARG
    assert decode(out=A + 1) == fd.FD_ERR_INVALID_ARG
    assert decode(out=A + 4) == fd.FD_ERR_INVALID_ARG
    assert decode(scale=float("inf")) == fd.FD_ERR_INVALID_ARG
    assert decode(scale=float("nan")) == fd.FD_ERR_INVALID_ARG
    assert decode(shape=(1, 4, 3, 4096, 128)) == fd.FD_ERR_INVALID_ARG
    assert decode(shape=(1, 4, 4, 4096, 80)) == fd.FD_ERR_UNSUPPORTED
    assert decode(n=-2) == fd.FD_ERR_INVALID_ARG
    # paged geometry without a table, and a table without geometry
    assert decode(page_size=16, max_pages_per_seq=256, num_pages=4) == fd.FD_ERR_INVALID_ARG
    assert decode(pt=A) == fd.FD_ERR_INVALID_ARG
    # a multi-split plan needs a big enough, aligned workspace
    assert decode() == fd.FD_ERR_WORKSPACE
    assert decode(workspace=A, workspace_bytes=100) == fd.FD_ERR_WORKSPACE
    need = fd.fd_workspace_bytes(1, 4, 4, 4096, 128, 16, opts())
    assert decode(workspace=A + 16, workspace_bytes=need) == fd.FD_ERR_WORKSPACE
    assert "workspace" in fd.fd_last_error()
    assert fd.fd_split(A, A, None, None, None, A, A, 1, 4, 4, 4096, 128, 0.1, 16, opts()) == fd.FD_ERR_INVALID_ARG
    assert fd.fd_combine(None, None, A, 1, 4, 4, 4096, 128, 16, opts()) == fd.FD_ERR_INVALID_ARG
    assert fd.fd_combine(None, A, A, 1, 4, 4, 4096, 128, 16, opts()) == fd.FD_ERR_WORKSPACE


def test_append_plans_cover_one_more_token(lib):
    for (B, Hq, Hkv, T, D) in [(1, 4, 4, 1024, 64), (2, 32, 8, 4096, 128), (1, 8, 8, 128, 128),
                               (3, 6, 2, 1000, 64), (1, 1, 1, 1, 128)]:
        for n in (0, 1, 4, 100000):
            st, p = plan(B, Hq, Hkv, T, D, n, flags=fd.FD_FLAG_APPEND)
            assert st == fd.FD_OK, fd.fd_last_error()
            assert p.chunk * p.n_splits >= T + 1 > p.chunk * (p.n_splits - 1)
    # paged: the stream plan does not depend on T
    st, p = plan(4, 8, 2, 4096, 128, 0, flags=fd.FD_FLAG_APPEND, page_size=16,
                 max_pages_per_seq=256, num_pages=10)
    assert st == fd.FD_OK and p.stream


@pytest.mark.parametrize("nq", [1, 2, 3, 8, 16])
def test_plan_several_queries(lib, nq):
    # the n_q queries of a kv head's group are rows of one block of work: the
    # matrix-core path once they make 4 rows, KV read once per head block
    for (G, dt) in [(1, fd.FD_F16), (2, fd.FD_BF16), (4, fd.FD_BF16), (8, fd.FD_F32)]:
        B, Hkv, T, D = 2, 2, 4096, 128
        st, p = plan(B, G * Hkv, Hkv, T, D, 0, dtype=dt, n_queries=nq)
        assert st == fd.FD_OK, fd.fd_last_error()
        R = nq * G
        if dt != fd.FD_F32 and R > 32:      # contiguous: the query-tiled kernel from 33 rows
            assert p.path == fd.FD_PATH_PREFILL
            continue
        want_mfma = dt != fd.FD_F32 and R >= 4
        assert p.path == (fd.FD_PATH_MFMA if want_mfma else fd.FD_PATH_VALU)
        assert p.heads_per_block * p.head_blocks >= R > p.heads_per_block * (p.head_blocks - 1)
        if want_mfma:
            assert p.heads_per_block == (32 if R > 16 else 16)
        if p.n_splits > 1:
            assert p.workspace_bytes >= B * nq * G * Hkv * p.n_splits * (D + 2) * 4
        st, p2 = plan(B, G * Hkv, Hkv, T, D, 0, dtype=dt, n_queries=nq, causal=1)
        assert st == fd.FD_OK and p2.n_splits == p.n_splits


def test_several_queries_rejects(lib):
    assert plan(1, 4, 4, 100, 128, n_queries=65537)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, n_queries=-1)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, n_queries=17, dtype=fd.FD_F32)[0] == fd.FD_ERR_UNSUPPORTED
    assert plan(1, 4, 4, 100, 128, n_queries=17, path=fd.FD_PATH_VALU)[0] == fd.FD_ERR_UNSUPPORTED
    assert plan(1, 4, 4, 100, 128, path=fd.FD_PATH_PREFILL, dtype=fd.FD_F32)[0] == fd.FD_ERR_UNSUPPORTED
    assert plan(1, 4, 4, 100, 128, path=5)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, n_queries=2, causal=2)[0] == fd.FD_ERR_INVALID_ARG
    assert plan(1, 4, 4, 100, 128, n_queries=0)[0] == fd.FD_OK          # 0 means one query
    st = plan(1, 4, 4, 100, 128, n_queries=2, flags=fd.FD_FLAG_APPEND)[0]
    assert st == fd.FD_ERR_UNSUPPORTED


def _query_tiled_splits(units, T, cus=256, n_req=0, tiles=2):
    """The planner's KV split rule for the query-tiled kernel, restated:
    about 8 * cus workgroups (four rounds at two per compute unit), none
    once the row tiles alone give 4 * cus; with one row tile per kv head of
    a contiguous cache 4 * cus, none from 2 * cus; no split below 1024
    tokens; chunks are whole 32-token tiles."""
    if n_req > 0:
        n = min(n_req, -(-T // 32))
    elif units >= (2 if tiles == 1 else 4) * cus:
        n = 1
    else:
        target = (8 if tiles > 1 else 4) * cus
        n = 1 if units >= target else min(-(-target // units), max(1, T // 1024))
    chunk = -(-(-(-T // n)) // 32) * 32
    return -(-T // chunk), chunk


@pytest.mark.parametrize("nq,G", [(17, 1), (100, 4), (4096, 8), (65536, 1)])
def test_plan_query_tiled(lib, nq, G):
    # more than 16 queries per sequence: one workgroup per 128 query rows of
    # each (sequence, kv head) and KV split; the KV axis is split only while
    # the row tiles leave the device short of workgroups.  bf16 takes a
    # workspace for V converted to f16 (scale exponents, chunk maxima,
    # transposed tiles; 256-byte aligned pieces), and with several splits
    # the partials follow it
    B, Hkv, T, D = 2, 2, 8192, 128
    a256 = lambda x: -(-x // 256) * 256
    sl = B * Hkv
    R = nq * G
    tiles = -(-R // 128)
    n, chunk = _query_tiled_splits(B * Hkv * tiles, T, tiles=tiles)
    parts = sl * R * n
    part_bytes = (a256(parts * D * 4) + 2 * a256(parts * 4)) if n > 1 else 0
    st, p = plan(B, G * Hkv, Hkv, T, D, 0, n_queries=nq, causal=1, dtype=fd.FD_F16)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.path == fd.FD_PATH_PREFILL and p.n_splits == n and p.workspace_bytes == part_bytes
    st, p = plan(B, G * Hkv, Hkv, T, D, 0, n_queries=nq, causal=1)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.path == fd.FD_PATH_PREFILL and p.n_splits == n
    # bf16 V is converted from 1024 query rows per kv head
    vt_bytes = a256(sl * 4) + a256(sl * (T // 256) * 4) + a256(sl * T * D * 2) if R >= 1024 else 0
    assert p.workspace_bytes == vt_bytes + part_bytes
    assert not p.fused and not p.stream and p.combine == (n > 1)
    assert (p.grid[0], p.grid[1], p.grid[2]) == (tiles * n, Hkv, B) and p.head_blocks == tiles
    if n > 1:
        assert p.chunk == chunk and p.chunk % 32 == 0 and (n - 1) * chunk < T
    # forced for a few queries too
    st, p = plan(B, G * Hkv, Hkv, T, D, 0, n_queries=2, path=fd.FD_PATH_PREFILL)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_PREFILL


@pytest.mark.parametrize("n_req", [1, 2, 5, 7, 300, 100000])
def test_plan_query_tiled_explicit_splits(lib, n_req):
    # an explicit split count is taken as asked, capped at one 32-token tile
    # per split; the effective count covers T with no empty split
    B, Hkv, G, T, D, nq = 1, 8, 4, 4000, 128, 512
    n, chunk = _query_tiled_splits(0, T, n_req=n_req, tiles=16)
    st, p = plan(B, G * Hkv, Hkv, T, D, n_req, n_queries=nq, causal=1)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.path == fd.FD_PATH_PREFILL and p.n_splits == n and p.combine == (n > 1)
    if n > 1:
        assert p.chunk == chunk and (n - 1) * chunk < T <= n * chunk
    assert p.grid[0] == 16 * n


def append(q=A, kn=A + 8192, vn=A + 16384, k=A, v=A, pt=None, sl=A, out=A, lse=A, shape=(1, 4, 4, 4096, 128),
           scale=0.1, n=16, **kw):
    return fd.fd_append_decode(q, kn, vn, k, v, pt, sl, out, lse, *shape, scale, n, opts(**kw))


def test_append_rejects_before_launch(lib):
    # FD_FLAG_APPEND plans are run by fd_append_decode only
    assert decode(flags=fd.FD_FLAG_APPEND) == fd.FD_ERR_INVALID_ARG
    assert "fd_append_decode" in fd.fd_last_error()
    assert fd.fd_split(A, A, A, None, None, A, A, 1, 4, 4, 4096, 128, 0.1, 16,
                       opts(flags=fd.FD_FLAG_APPEND)) == fd.FD_ERR_INVALID_ARG
    assert fd.fd_combine(None, A, A, 1, 4, 4, 4096, 128, 16,
                         opts(flags=fd.FD_FLAG_APPEND)) == fd.FD_ERR_INVALID_ARG
    assert append(kn=None) == fd.FD_ERR_INVALID_ARG
    assert append(vn=None) == fd.FD_ERR_INVALID_ARG
    assert append(kn=MIS) == fd.FD_ERR_INVALID_ARG
    assert append(k=A + 4096, kn=A + 4096) == fd.FD_ERR_INVALID_ARG     # k_new is the cache
    assert append(q=None) == fd.FD_ERR_INVALID_ARG
    assert append() == fd.FD_ERR_WORKSPACE                             # 16 splits need a workspace
    need = fd.fd_workspace_bytes(1, 4, 4, 4096, 128, 16, opts(flags=fd.FD_FLAG_APPEND))
    st, p = plan(1, 4, 4, 4096, 128, 16, flags=fd.FD_FLAG_APPEND)
    assert st == fd.FD_OK and need == p.workspace_bytes > 0
    assert append(workspace=A, workspace_bytes=need - 256) == fd.FD_ERR_WORKSPACE


def test_status_strings(lib):
    for st in range(5):
        assert fd.fd_status_string(st).startswith("FD_")
    assert "unknown" in fd.fd_status_string(99)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_reports_hip_error(lib):
    # Planning for the current device needs one: without a GPU this fails
    # cleanly instead of launching.
    need = 1 << 30
    st = decode(num_cus=0, workspace=A, workspace_bytes=need)
    assert st == fd.FD_ERR_HIP
    assert "hip" in fd.fd_last_error().lower()


def test_plan_query_tiled_size_limits(lib):
    # bf16 query-tiled plans address each (batch, kv head) of converted V with
    # 32-bit offsets: a paged T whose converted slice reaches 4 GiB is refused
    T = (1 << 24)                                   # 2^24 tokens x 128 x 2 B = 4 GiB
    kw = dict(n_queries=256, page_size=16, max_pages_per_seq=T // 16, num_pages=1)   # 1024 rows: V converted
    st, _ = plan(1, 8, 2, T, 128, 0, **kw)
    assert st == fd.FD_ERR_UNSUPPORTED and "4 GiB" in fd.fd_last_error()
    st, _ = plan(1, 8, 2, T - 64, 128, 0, **kw)
    assert st == fd.FD_OK, fd.fd_last_error()
    st, p = plan(1, 8, 2, T, 128, 1, dtype=fd.FD_F16, **kw)   # f16 needs no conversion
    assert st == fd.FD_OK and p.n_splits == 1 and p.workspace_bytes == 0
    st, p = plan(1, 8, 2, T, 128, 0, dtype=fd.FD_F16, **kw)   # eight row tiles: the KV axis is split
    assert st == fd.FD_OK and p.n_splits == 128 and p.workspace_bytes > 0


@pytest.mark.parametrize("nq,G,dtype,want", [
    (1, 16, fd.FD_BF16, fd.FD_PATH_MFMA),        # 16 rows: split kernels
    (1, 32, fd.FD_BF16, fd.FD_PATH_MFMA),        # 32 rows: two row blocks of the split kernel
    (1, 64, fd.FD_BF16, fd.FD_PATH_PREFILL),     # 64 rows of one query
    (4, 4, fd.FD_F16, fd.FD_PATH_MFMA),
    (5, 4, fd.FD_BF16, fd.FD_PATH_MFMA),         # 20 rows
    (8, 4, fd.FD_F16, fd.FD_PATH_MFMA),          # 32 rows
    (9, 4, fd.FD_F16, fd.FD_PATH_PREFILL),       # 36 rows
    (16, 8, fd.FD_BF16, fd.FD_PATH_PREFILL),
    (16, 8, fd.FD_F32, fd.FD_PATH_VALU),         # fp32 stays on the vector kernel
    (17, 1, fd.FD_F16, fd.FD_PATH_PREFILL),      # more than 16 queries
])
def test_plan_rows_route(lib, nq, G, dtype, want):
    # query rows per kv head (n_q * G) past 32 take the query-tiled kernel,
    # which reads K/V once for a 64- or 128-row tile, contiguous or paged;
    # one-query calls with an appended token stay on the split kernels
    st, p = plan(2, G * 2, 2, 4096, 128, 0, n_queries=nq, causal=1 if nq > 1 else 0, dtype=dtype)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.path == want
    st, p = plan(2, G * 2, 2, 4096, 128, 0, n_queries=nq, causal=1 if nq > 1 else 0, dtype=dtype,
                 page_size=16, max_pages_per_seq=256, num_pages=10)
    assert st == fd.FD_OK, fd.fd_last_error()
    assert p.path == want
    st, p = plan(2, 64 * 2, 2, 4096, 128, 0, flags=fd.FD_FLAG_APPEND)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_MFMA


def test_plan_query_tiled_paged_splits(lib, monkeypatch):
    # a paged (ragged) batch with one row tile per kv head is planned for
    # four rounds of workgroups, a contiguous one for two; with the chunk
    # chosen on the device from the lengths (the default for such ordered
    # calls) the plan holds twice the columns and the smallest chunk
    B, Hq, Hkv, T = 16, 32, 8, 65536
    kw = dict(n_queries=16, causal=1)
    paged = dict(page_size=16, max_pages_per_seq=T // 16, num_pages=10)
    monkeypatch.setenv("FD_PREFILL_DEVCHUNK", "0")
    st, p = plan(B, Hq, Hkv, T, 128, 0, **paged, **kw)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_PREFILL
    assert p.n_splits == _query_tiled_splits(B * Hkv, T, tiles=2)[0] == 16 and p.chunk == 4096
    monkeypatch.delenv("FD_PREFILL_DEVCHUNK")
    st, p = plan(B, Hq, Hkv, T, 128, 0, **paged, **kw)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_PREFILL and p.n_splits == 32 and p.chunk == 2048
    st, p = plan(B, Hq, Hkv, T, 128, 5, **paged, **kw)          # an explicit count is kept
    assert st == fd.FD_OK and p.n_splits == 5
    st, p = plan(B, Hq, Hkv, T, 128, 0, **kw)
    assert st == fd.FD_OK and p.n_splits == _query_tiled_splits(B * Hkv, T, tiles=1)[0] == 8
    # one row tile per kv head that already gives two workgroups per CU: no split
    st, p = plan(64, 64, 8, 32768, 128, 0, n_queries=8, causal=1)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_PREFILL and p.n_splits == 1 and p.workspace_bytes == 0
    st, p = plan(32, 64, 8, 32768, 128, 0, n_queries=8, causal=1)
    assert st == fd.FD_OK and p.n_splits == _query_tiled_splits(32 * 8, 32768, tiles=1)[0] == 4


_LOG_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
from split_kv_fd_amd import fd
o = fd.fd_options_t(); fd.fd_options_init(o); o.num_cus = 256
p = fd.fd_plan_t()
assert fd.fd_plan(4, 32, 8, 131072, 128, 0, o, p) == fd.FD_OK
print("PLAN", p.path, p.n_splits, p.chunk, p.fused, p.stream, flush=True)
o.page_size, o.max_pages_per_seq, o.num_pages = 16, 4096, 100
assert fd.fd_plan(16, 32, 8, 65536, 128, 0, o, p) == fd.FD_OK
print("PLAN", p.path, p.n_splits, p.chunk, p.fused, p.stream, flush=True)
o.n_queries, o.causal = 16, 1
assert fd.fd_plan(16, 32, 8, 65536, 128, 0, o, p) == fd.FD_OK
print("PLAN", p.path, p.n_splits, p.chunk, p.fused, p.stream, flush=True)
o.n_queries, o.causal, o.page_size = 1, 0, 0
# fails validation: nothing is planned, nothing logged
assert fd.fd_decode(None, 1 << 20, 1 << 20, None, None, 1 << 20, None, 1, 4, 4, 4096, 128, 0.1, 0, o) != fd.FD_OK
"""


@pytest.mark.parametrize("flag", ["1", None])
def test_fd_log_prints_each_plan(lib, flag):
    # FD_LOG=1: one stderr line per planned call naming the path and the plan
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("FD_LOG", None)
    if flag:
        env["FD_LOG"] = flag
    r = subprocess.run([sys.executable, "-c", _LOG_SCRIPT, ROOT], capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    plans = [ln.split()[1:] for ln in r.stdout.splitlines() if ln.startswith("PLAN")]
    logs = [ln for ln in r.stderr.splitlines() if ln.startswith("[fd] ")]
    if not flag:
        assert logs == []
        return
    assert len(logs) == 3 and all(ln.startswith("[fd] fd_plan ") for ln in logs)
    names = {0: "valu", 1: "mfma", 2: "query-tiled"}
    for ln, (path, n, chunk, fused, stream) in zip(logs, plans):
        kv = dict(t.split("=", 1) for t in ln.split() if "=" in t)
        assert kv["path"] == names[int(path)] and kv["n_splits"] == n and kv["chunk"] == chunk
        assert kv["stream"] == stream
        assert kv["merge"] == ("none" if int(n) == 1 else "fused" if (int(fused) or int(stream)) else "combine-kernel")
    assert "paged=1" in logs[1] and "stream=1" in logs[1] and "B=16" in logs[1]
    # a ragged paged few-query call: the order pass picks the split size
    assert "n_queries=16" in logs[2] and "chunk_on_device=1" in logs[2]
    assert "chunk_on_device=0" in logs[0] and "chunk_on_device=0" in logs[1]


def noalloc(q=A, k=A, v=A, pt=None, sl=None, out=A, lse=A, shape=(1, 4, 4, 4096, 128), scale=0.1,
            n=16, **kw):
    return fd.fd_decode_noalloc(q, k, v, pt, sl, out, lse, *shape, scale, n, opts(**kw))


def test_noalloc_rejects_before_device_work(lib):
    # the static scratch replaces the caller's workspace: passing one is an error
    assert noalloc(workspace=A, workspace_bytes=1 << 20) == fd.FD_ERR_INVALID_ARG
    assert "workspace must be NULL" in fd.fd_last_error()
    # argument checks as fd_decode, all before the device is touched
    assert noalloc(q=None) == fd.FD_ERR_INVALID_ARG
    assert noalloc(k=MIS) == fd.FD_ERR_INVALID_ARG
    assert noalloc(out=A + 4) == fd.FD_ERR_INVALID_ARG
    assert noalloc(scale=float("nan")) == fd.FD_ERR_INVALID_ARG
    assert noalloc(pt=A) == fd.FD_ERR_INVALID_ARG
    assert noalloc(shape=(1, 4, 4, 4096, 80)) == fd.FD_ERR_UNSUPPORTED
    # a plan needing more than the scratch holds is refused with the sizes
    kw = dict(page_size=16, max_pages_per_seq=4096, num_pages=100)
    st, p = plan(2048, 32, 8, 65536, 128, 0, **kw)
    assert st == fd.FD_OK and p.workspace_bytes > fd.FD_NOALLOC_SCRATCH_BYTES
    assert noalloc(shape=(2048, 32, 8, 65536, 128), pt=A, sl=A, n=0, **kw) == fd.FD_ERR_WORKSPACE
    msg = fd.fd_last_error()
    assert str(p.workspace_bytes) in msg and str(fd.FD_NOALLOC_SCRATCH_BYTES) in msg
    # bf16 prefill that converts V needs about V's size: refused too
    st, p = plan(4, 32, 8, 4096, 128, 0, n_queries=4096)
    assert st == fd.FD_OK and p.workspace_bytes > fd.FD_NOALLOC_SCRATCH_BYTES
    assert noalloc(shape=(4, 32, 8, 4096, 128), n=0, n_queries=4096) == fd.FD_ERR_WORKSPACE


def test_noalloc_scratch_fits_the_decode_workloads(lib):
    # every decode workload's automatic plan fits the static scratch
    for name in ("tiny_f32", "mha32k_f16", "gqa128k_bf16", "paged_ragged_bf16", "gqa_b64_bf16"):
        s = SPECS[name]
        dt = {"f32": fd.FD_F32, "f16": fd.FD_F16, "bf16": fd.FD_BF16}[s.dtype]
        kw = dict(page_size=16, max_pages_per_seq=4096, num_pages=100) if s.paged else {}
        st, p = plan(s.B, s.Hq, s.Hkv, s.T, s.D, s.n_splits, dtype=dt, **kw)
        assert st == fd.FD_OK and p.workspace_bytes <= fd.FD_NOALLOC_SCRATCH_BYTES, (name, p.workspace_bytes)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_noalloc_without_device_reports_hip_error(lib):
    # a valid call that fits reaches the device lookup, which fails cleanly here
    assert noalloc(n=0) == fd.FD_ERR_HIP


def test_plan_query_tiled_column_order_workspace(lib):
    # ragged paged calls with one row tile per kv head and several splits
    # reserve B * n_splits order entries after the partials, then 256 bytes
    # for the chunk the order pass picks; contiguous caches, several row
    # tiles or more than 1024 sequences do not
    kw = dict(n_queries=16, page_size=16, max_pages_per_seq=4096, num_pages=100)
    st, p = plan(16, 32, 8, 65536, 128, 0, **kw)
    assert st == fd.FD_OK and p.path == fd.FD_PATH_PREFILL and p.head_blocks == 1 and p.n_splits > 1
    parts = 16 * 8 * 64 * p.n_splits
    a256 = lambda x: -(-x // 256) * 256
    want = a256(parts * 128 * 4) + 2 * a256(parts * 4)
    assert p.workspace_bytes == want + a256(16 * p.n_splits * 4) + 256
    st, c = plan(16, 32, 8, 65536, 128, 0, n_queries=16)
    assert st == fd.FD_OK and c.workspace_bytes == a256(16 * 8 * 64 * c.n_splits * 128 * 4) + 2 * a256(16 * 8 * 64 * c.n_splits * 4)
    st, big = plan(1100, 32, 8, 2048, 128, 4, **dict(kw, max_pages_per_seq=128))
    parts = 1100 * 8 * 64 * big.n_splits
    assert st == fd.FD_OK and big.workspace_bytes == a256(parts * 128 * 4) + 2 * a256(parts * 4)
