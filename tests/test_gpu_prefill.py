"""GPU parity of the query-tiled kernel (many queries per sequence: the
prefill phase) against the oracle's per-query decode, causal or not."""
import pytest
import torch

from oracle import oracle as oracle_mod
from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity
from tests.test_gpu_multi import check_multi, contiguous

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G,dtype,D", [(1, "bf16", 128), (4, "bf16", 128), (8, "f16", 128), (4, "f16", 64),
                                       (2, "bf16", 64)])
def test_prefill_contiguous(causal, G, dtype, D):
    # prompts with and without a cached prefix, a sequence shorter than the
    # query count (early queries see nothing when causal), an empty one
    Hkv = 2
    nq = 100
    case = contiguous("mha32k_f16", [300, 100, 37, 0, 257], Hq=G * Hkv, Hkv=Hkv, T=300, D=D, dtype=dtype)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    plan = check_multi(case, q, causal, what=f"prefill G={G} {dtype} D={D} causal={causal}")
    assert plan["path"] == "prefill" and plan["n_splits"] == 1


@pytest.mark.parametrize("nq", [17, 64, 65, 256])
def test_prefill_query_counts(nq):
    # row tiles with a ragged last tile, and tiles that cross query boundaries
    case = contiguous("gqa128k_bf16", [700, 512], Hq=12, Hkv=2, T=700)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    check_multi(case, q, True, what=f"prefill nq={nq}")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_paged(causal):
    for P in (1, 16, 256):
        s = inputs.spec("paged_ragged_bf16", B=3, Hq=8, Hkv=2, T=900, page_size=P, len_lo=50, len_hi=900)
        case = inputs.make_case(s).to(DEV)
        q = inputs.make_q_multi(s, 48).to(DEV)
        plan = check_multi(case, q, causal, what=f"prefill paged P={P} causal={causal}")
        assert plan["path"] == "prefill"


@pytest.mark.parametrize("nq", [1, 3, 16])
def test_prefill_kernel_for_few_queries(nq):
    # the query-tiled kernel forced on few queries agrees with the oracle and
    # with the split-KV kernels
    case = contiguous("gqa128k_bf16", [2000, 1000, 5], Hq=16, Hkv=4, T=2000)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    check_multi(case, q, True, path="prefill", what=f"forced prefill nq={nq}")
    a = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=True, path="prefill")
    out_a, lse_a = (x.clone() for x in a())
    d = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=True)
    out_d, lse_d = d()
    torch.cuda.synchronize()
    # the query-tiled kernel rounds P to f16 (weights within 2^-11), the
    # split kernels keep it in fp32: outputs agree within 1e-3 of max|V|,
    # the lse (summed in fp32 on both) within 1e-4
    vmax = float(case.v.float().abs().max())
    assert torch.allclose(out_a, out_d, rtol=0, atol=1e-3 * vmax)
    assert torch.allclose(lse_a, lse_d, rtol=0, atol=1e-4)


def test_prefill_full_size_every_query():
    # a 2048-token prompt after a 2048-token prefix, GQA 32/8, bf16: every
    # query and head of both sequences against the oracle
    s = inputs.spec("gqa128k_bf16", B=2, T=4096)
    case = inputs.make_case(s, device=DEV)
    nq = 2048
    q = inputs.make_q_multi(s, nq, device=DEV)
    dec = Decoder(q, case.k, case.v, scale=s.scale, causal=True)
    assert dec.plan["path"] == "prefill"
    parity.announce(f"prefill full size nq={nq} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    parity.all_queries(case, q, out.cpu().double().numpy(), lse.cpu().double().numpy(), [0, 1], True,
                       f"prefill full size nq={nq}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.35])
def test_prefill_scale_sign(scale):
    # the scale enters the exponent on unmasked tiles: negative and zero
    # scales must give the oracle's softmax too
    case = contiguous("gqa128k_bf16", [300, 129], Hq=8, Hkv=2, T=300)
    q = inputs.make_q_multi(case.spec, 40).to(DEV)
    host = case.to("cpu")
    for causal in (False, True):
        ref_out, ref_lse = oracle_mod.default().decode_multi(q.cpu(), host.k, host.v, scale, causal=causal,
                                                             seq_lens=host.seq_lens)
        dec = Decoder(q, case.k, case.v, scale=scale, seq_lens=case.seq_lens, causal=causal)
        assert dec.plan["path"] == "prefill"
        parity.announce(f"prefill scale={scale} causal={causal}")
        out, lse = dec()
        torch.cuda.synchronize()
        parity.compare(case, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(host), f"prefill scale={scale} causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_prefill_sharp_softmax(dtype, scale):
    # large scales spread the logits over tens of log2 units: most
    # probabilities are tiny (an f16 P formed without headroom would fall
    # into the subnormal range) and the running max moves often
    case = contiguous("gqa128k_bf16", [640, 333], Hq=8, Hkv=2, T=640, dtype=dtype)
    q = inputs.make_q_multi(case.spec, 64).to(DEV)
    host = case.to("cpu")
    for causal in (False, True):
        ref_out, ref_lse = oracle_mod.default().decode_multi(q.cpu(), host.k, host.v, scale, causal=causal,
                                                             seq_lens=host.seq_lens)
        dec = Decoder(q, case.k, case.v, scale=scale, seq_lens=case.seq_lens, causal=causal)
        assert dec.plan["path"] == "prefill"
        parity.announce(f"prefill sharp dtype={dtype} scale={scale} causal={causal}")
        out, lse = dec()
        torch.cuda.synchronize()
        parity.compare(case, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(host), f"prefill sharp dtype={dtype} scale={scale} causal={causal}")


def test_prefill_full_size_f16_every_query():
    # MHA 32 heads, f16 (one P product per tile): a 4096-token causal
    # prompt; every query of four of the heads against the oracle
    s = inputs.spec("mha32k_f16", B=1, T=4096)
    case = inputs.make_case(s, device=DEV)
    nq = 4096
    q = inputs.make_q_multi(s, nq, device=DEV)
    dec = Decoder(q, case.k, case.v, scale=s.scale, causal=True)
    assert dec.plan["path"] == "prefill"
    parity.announce(f"prefill f16 full size nq={nq} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    parity.all_queries(case, q, out.cpu().double().numpy(), lse.cpu().double().numpy(), [0], True,
                       f"prefill f16 full size nq={nq}", heads=[0, 9, 22, 31])


@pytest.mark.parametrize("vt", ["1", "0"])
@pytest.mark.parametrize("vmul", [2.0 ** 20, 2.0 ** -20, 2.0 ** -130, 0.0])
def test_prefill_bf16_value_range(env_switch, vt, vmul):
    # bf16 V far from 1 in magnitude -- large, small, in the bf16 subnormal
    # range, all zero: the per-(sequence, kv head) scale of the f16
    # conversion (vt = 1; forced, as 160 query rows would not convert) keeps
    # the value product within the tolerance of max|V|, and so does the
    # two-part bf16 probability product (vt = 0)
    env_switch.setenv("FD_PREFILL_VT", vt)
    case = contiguous("gqa128k_bf16", [300, 129], Hq=8, Hkv=2, T=300)
    case.v = (case.v.float() * vmul).to(torch.bfloat16)
    q = inputs.make_q_multi(case.spec, 40).to(DEV)
    host = case.to("cpu")
    for causal in (False, True):
        ref_out, ref_lse = oracle_mod.default().decode_multi(q.cpu(), host.k, host.v, case.spec.scale,
                                                             causal=causal, seq_lens=host.seq_lens)
        dec = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=causal)
        assert dec.plan["path"] == "prefill" and (dec.plan["workspace_bytes"] > 0) == (vt == "1")
        parity.announce(f"prefill bf16 V x {vmul:g} vt={vt} causal={causal}")
        out, lse = dec()
        torch.cuda.synchronize()
        parity.compare(case, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(host), f"prefill bf16 V x {vmul:g} causal={causal}")


@pytest.fixture
def env_switch(monkeypatch):
    # the library reads its FD_* switches when a call is prepared
    return monkeypatch


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_bf16_split_p_form(env_switch, causal):
    # FD_PREFILL_VT=0: bf16 V read as given, P in a high and a low bf16 part
    # (no workspace) -- the same oracle bar, contiguous and paged
    env_switch.setenv("FD_PREFILL_VT", "0")
    case = contiguous("gqa128k_bf16", [300, 100, 0], Hq=8, Hkv=2, T=300)
    q = inputs.make_q_multi(case.spec, 48).to(DEV)
    plan = check_multi(case, q, causal, what=f"prefill bf16 split P causal={causal}")
    assert plan["path"] == "prefill" and plan["workspace_bytes"] == 0
    s = inputs.spec("paged_ragged_bf16", B=3, Hq=8, Hkv=2, T=900, page_size=16, len_lo=50, len_hi=900)
    pc = inputs.make_case(s).to(DEV)
    check_multi(pc, inputs.make_q_multi(s, 40).to(DEV), causal, what=f"prefill bf16 split P paged causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n_splits", [0, 2])
def test_prefill_work_order_does_not_change_results(env_switch, dtype, n_splits):
    # the XCD-aware work orders only permute which workgroup takes which
    # (sequence, kv head, split, row tile): outputs are bit-identical.  24
    # (48 split) ranges: 3 (6) per XCD, so the causal pairs end on a single
    # range (or not), 5 row tiles each
    case = contiguous("gqa128k_bf16", [700, 333, 512], Hq=16, Hkv=8, T=700, dtype=dtype)
    q = inputs.make_q_multi(case.spec, 300).to(DEV)
    res = []
    for x, pairs in (("0", "1"), ("1", "0"), ("1", "2")):       # plain, ranges in turn, in pairs
        env_switch.setenv("FD_PREFILL_XCD", x)
        env_switch.setenv("FD_PREFILL_PAIRS", pairs)
        dec = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=True,
                      n_splits=n_splits)
        assert dec.plan["path"] == "prefill" and dec.plan["head_blocks"] == 5
        out, lse = dec()
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    for out, lse in res[1:]:
        assert torch.equal(out, res[0][0]) and torch.equal(lse, res[0][1])
    check_multi(case, q, True, n_splits=n_splits, what=f"paired causal order {dtype} n={n_splits}")


def test_prefill_full_prompt_causal_pairs():
    # causal queries covering the whole cache take the paired order by
    # default (MHA, 64 ranges: 8 per XCD, 8 row tiles each); the oracle on
    # every row
    case = contiguous("mha32k_f16", [1024, 1000], Hq=32, Hkv=32, T=1024)
    q = inputs.make_q_multi(case.spec, 1024).to(DEV)
    plan = check_multi(case, q, True, what="full-prompt causal, paired order")
    assert plan["path"] == "prefill" and plan["head_blocks"] == 8


# ------------------------------------------------------------------ KV splits of the query-tiled kernel

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
@pytest.mark.parametrize("n", [2, 3, 7, 64])
def test_prefill_kv_splits(causal, dtype, D, n):
    # the KV axis split n ways (chunks of whole 32-token tiles; the last
    # split short, some splits past a short sequence's end or past what a
    # causal row tile sees), partials merged by the combine kernel; an empty
    # sequence and one shorter than the query count.  The workspace starts
    # as 0xFF bytes (NaN partials): a merge that read an unwritten split
    # would show
    case = contiguous("gqa128k_bf16", [1500, 37, 0, 777, 1200], Hq=8, Hkv=2, T=1500, D=D, dtype=dtype)
    q = inputs.make_q_multi(case.spec, 150).to(DEV)
    plan = check_multi(case, q, causal, n_splits=n, what=f"prefill splits n={n} {dtype} D={D} causal={causal}")
    chunk = -(-(-(-1500 // n)) // 32) * 32          # whole tiles: 64 asked gives 47 splits of 32 tokens
    assert plan["path"] == "prefill" and plan["n_splits"] == -(-1500 // chunk) and plan["combine"]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [3, 7])
def test_prefill_kv_splits_converted_v(env_switch, causal, n):
    # bf16 V converted to f16 (forced: 600 query rows would not convert):
    # each split's partial undoes the conversion scale before the merge
    env_switch.setenv("FD_PREFILL_VT", "1")
    case = contiguous("gqa128k_bf16", [1500, 37, 0, 777, 1200], Hq=8, Hkv=2, T=1500)
    q = inputs.make_q_multi(case.spec, 150).to(DEV)
    plan = check_multi(case, q, causal, n_splits=n, what=f"prefill splits converted V n={n} causal={causal}")
    assert plan["path"] == "prefill" and plan["n_splits"] == n and plan["workspace_bytes"] > 0


@pytest.mark.parametrize("nq,G,dtype", [(1, 64, "bf16"), (2, 20, "f16"), (9, 4, "bf16"), (16, 8, "bf16"),
                                         (1, 33, "bf16"), (5, 8, "f16"), (12, 4, "bf16")])
def test_many_rows_take_query_tiled_kernel(nq, G, dtype):
    # more than 32 query rows per kv head (n_q * G) of a contiguous cache go
    # to the query-tiled kernel, which reads K/V once for a 64- or 128-row
    # tile (bf16 V unconverted at these row counts); ragged lengths, one
    # empty sequence, both masks
    case = contiguous("gqa128k_bf16", [3000, 1500, 0], Hq=G * 2, Hkv=2, T=3000, dtype=dtype)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    for causal in ((False, True) if nq > 1 else (False,)):
        plan = check_multi(case, q, causal, what=f"many rows nq={nq} G={G} {dtype} causal={causal}")
        assert plan["path"] == "prefill" and plan["workspace_bytes"] >= 0
        # 64-row tiles (one 16-row block per wave) up to 64 rows, else 128
        assert plan["heads_per_block"] == (64 if nq * G <= 64 else 128)
        if dtype == "bf16" and plan["n_splits"] == 1:
            assert plan["workspace_bytes"] == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_small_and_large_row_tiles_agree(env_switch, dtype):
    # the 64-row and 128-row tiles both meet the oracle's bar on the same
    # rows (one tile holds every row here); they group rows into waves
    # differently, and a wave shares its masks and running-max moves, so
    # their rounding differs: they agree within 1e-3 of max|V| (f16
    # probabilities) and 1e-4 in the lse
    case = contiguous("gqa128k_bf16", [2500, 700, 1], Hq=16, Hkv=2, T=2500, dtype=dtype)
    q = inputs.make_q_multi(case.spec, 6).to(DEV)
    res = []
    for small in ("1", "0"):
        env_switch.setenv("FD_PREFILL_SMALL", small)
        plan = check_multi(case, q, True, n_splits=3, what=f"row tiles small={small} {dtype}")
        assert plan["path"] == "prefill" and plan["heads_per_block"] == (64 if small == "1" else 128)
        dec = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=True, n_splits=3)
        out, lse = dec()
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    vmax = float(case.v.float().abs().max())
    assert torch.allclose(res[0][0], res[1][0], rtol=0, atol=1e-3 * vmax)
    assert torch.allclose(res[0][1], res[1][1], rtol=0, atol=1e-4)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_kv_splits_paged(causal):
    for P in (1, 16, 256):
        s = inputs.spec("paged_ragged_bf16", B=3, Hq=8, Hkv=2, T=2000, page_size=P, len_lo=50, len_hi=2000)
        case = inputs.make_case(s).to(DEV)
        q = inputs.make_q_multi(s, 48).to(DEV)
        for n in (2, 5):
            plan = check_multi(case, q, causal, n_splits=n, what=f"prefill splits paged P={P} n={n} causal={causal}")
            assert plan["path"] == "prefill" and plan["n_splits"] == n


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_kv_splits_split_p_form(env_switch, causal):
    # bf16 V read as given (P in two bf16 parts, no conversion): the
    # partials carry no conversion scale and no probability bias
    env_switch.setenv("FD_PREFILL_VT", "0")
    case = contiguous("gqa128k_bf16", [1000, 300, 0], Hq=8, Hkv=2, T=1000)
    q = inputs.make_q_multi(case.spec, 64).to(DEV)
    plan = check_multi(case, q, causal, n_splits=4, what=f"prefill splits bf16 split P causal={causal}")
    assert plan["path"] == "prefill" and plan["n_splits"] == 4


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_auto_splits_few_queries_long_cache(dtype):
    # 64 queries after an 8k-token prefix: one row tile per kv head, so the
    # planner splits the KV axis (a chunked-prefill step)
    case = contiguous("gqa128k_bf16", [8192, 5000], Hq=8, Hkv=2, T=8192, dtype=dtype)
    q = inputs.make_q_multi(case.spec, 64).to(DEV)
    for causal in (False, True):
        plan = check_multi(case, q, causal, what=f"prefill auto splits {dtype} causal={causal}")
        assert plan["path"] == "prefill" and plan["n_splits"] > 1


@pytest.mark.parametrize("scale", [-0.3, 2.0])
def test_prefill_kv_splits_scale(scale):
    # negative scales (folded into q) and sharp softmaxes, whose running
    # maxima differ much between splits, through the merge
    case = contiguous("gqa128k_bf16", [1100, 400], Hq=8, Hkv=2, T=1100)
    q = inputs.make_q_multi(case.spec, 40).to(DEV)
    host = case.to("cpu")
    for causal in (False, True):
        ref_out, ref_lse = oracle_mod.default().decode_multi(q.cpu(), host.k, host.v, scale, causal=causal,
                                                             seq_lens=host.seq_lens)
        dec = Decoder(q, case.k, case.v, scale=scale, seq_lens=case.seq_lens, causal=causal, n_splits=6)
        assert dec.plan["path"] == "prefill" and dec.plan["n_splits"] == 6
        parity.announce(f"prefill splits scale={scale} causal={causal}")
        out, lse = dec()
        torch.cuda.synchronize()
        parity.compare(case, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(host), f"prefill splits scale={scale} causal={causal}")


def test_prefill_kv_splits_separate_entry_points():
    # fd_split then fd_combine give fd_decode's result bit for bit, and the
    # same plan run twice gives identical bits
    case = contiguous("gqa128k_bf16", [900, 450], Hq=8, Hkv=2, T=900)
    q = inputs.make_q_multi(case.spec, 80).to(DEV)
    dec = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, causal=True, n_splits=3)
    out_a, lse_a = (x.clone() for x in dec())
    dec.out.fill_(float("nan"))
    dec.lse.fill_(float("nan"))
    dec.split()
    dec.combine()
    torch.cuda.synchronize()
    assert torch.equal(out_a, dec.out) and torch.equal(lse_a, dec.lse)
    out_c, lse_c = dec()
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_c) and torch.equal(lse_a, lse_c)


def test_prefill_ragged_full_size_every_query():
    # the paged ragged workload's shape (16-token pages, lengths from 1k to
    # 64k) with 512 causal queries per sequence, B=4: the automatic plan
    # splits the KV axis.  Every query of the shortest sequence (all heads)
    # and of the longest (two kv groups, 8 heads) against the oracle
    s = inputs.spec("paged_ragged_bf16", B=4)
    case = inputs.make_case(s, device=DEV)
    nq = 512
    q = inputs.make_q_multi(s, nq, device=DEV)
    dec = Decoder(q, case.k, case.v, scale=s.scale, page_table=case.page_table, seq_lens=case.seq_lens,
                  T=s.T, causal=True)
    assert dec.plan["path"] == "prefill" and dec.plan["n_splits"] > 1
    parity.announce(f"prefill ragged full size nq={nq} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    lens = case.lengths()
    out_h, lse_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    shortest = min(range(s.B), key=lambda b: lens[b])
    longest = max(range(s.B), key=lambda b: lens[b])
    parity.all_queries(case, q, out_h, lse_h, [shortest], True, f"prefill ragged T_b={lens[shortest]}")
    parity.all_queries(case, q, out_h, lse_h, [longest], True, f"prefill ragged T_b={lens[longest]}",
                       heads=[0, s.Hq - 1])


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("P", [1, 16, 64])
@pytest.mark.parametrize("nq,G,dtype", [(16, 4, "bf16"), (9, 4, "f16"), (40, 4, "f16"), (40, 4, "bf16")])
def test_query_tiled_paged_page_ids(P, nq, G, dtype, D):
    # paged caches through the query-tiled kernel in each page-id form: read
    # one tile ahead (64-row tiles; bf16 128-row tiles with V unconverted)
    # or just before (f16 128-row tiles); one-token pages take a page id
    # per token.  Ragged lengths, a page shuffle, KV splits, both masks
    s = inputs.spec("paged_ragged_bf16", B=3, Hq=G * 2, Hkv=2, T=1800, page_size=P, len_lo=40, len_hi=1800,
                    dtype=dtype, D=D)
    case = inputs.make_case(s).to(DEV)
    q = inputs.make_q_multi(s, nq).to(DEV)
    for causal in (False, True):
        for n in (0, 3):
            plan = check_multi(case, q, causal, n_splits=n,
                               what=f"paged page ids D={D} P={P} nq={nq} G={G} {dtype} n={n} causal={causal}")
            assert plan["path"] == "prefill"
            assert plan["heads_per_block"] == (64 if nq * G <= 64 else 128)


@pytest.mark.parametrize("n_splits", [0, 3, 7])
def test_query_tiled_column_order(env_switch, n_splits):
    # ragged paged calls with one row tile per kv head run their (sequence,
    # split) columns longest first: the order only permutes which workgroup
    # takes which column, so results are bit-identical to the plain order,
    # and meet the oracle.  Lengths include an empty sequence, an exact
    # multiple of the chunk, one shorter than a chunk and the longest.
    s = inputs.spec("paged_ragged_bf16", B=6, Hq=8, Hkv=2, T=5000, page_size=16, len_lo=0, len_hi=5000)
    case = inputs.make_case(s)
    case.seq_lens[:] = torch.tensor([4096, 0, 5000, 700, 2048, 3333], dtype=torch.int32)
    case = case.to(DEV)
    q = inputs.make_q_multi(s, 16).to(DEV)
    res = []
    env_switch.setenv("FD_PREFILL_DEVCHUNK", "0")          # the plan's chunk both ways
    for order in ("1", "0"):
        env_switch.setenv("FD_PREFILL_ORDER", order)
        plan = check_multi(case, q, True, n_splits=n_splits, what=f"column order={order} n={n_splits}")
        assert plan["path"] == "prefill" and plan["head_blocks"] == 1 and plan["n_splits"] > 1
        dec = Decoder(q, case.k, case.v, scale=s.scale, page_table=case.page_table, seq_lens=case.seq_lens,
                      T=s.T, causal=True, n_splits=n_splits)
        dec.workspace.fill_(0xFF)
        out, lse = dec()
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("dtype,D,nq", [("bf16", 128, 16), ("f16", 128, 16), ("bf16", 64, 16), ("bf16", 128, 40)])
def test_query_tiled_pool_offsets_agree(env_switch, dtype, D, nq):
    # paged pools under 4 GiB are addressed with 32-bit byte offsets into a
    # buffer resource; the 64-bit row addressing (FD_PREFILL_POOL32=0) loads
    # the same rows, so the results are bit-identical, and both meet the
    # oracle.  64-row tiles (V stored as loaded, transposing reads, three
    # workgroups per CU) and 128-row tiles; 16-token pages, shuffled pool
    s = inputs.spec("paged_ragged_bf16", B=4, Hq=8, Hkv=2, D=D, T=3000, page_size=16, len_lo=0, len_hi=3000,
                    dtype=dtype)
    case = inputs.make_case(s).to(DEV)
    q = inputs.make_q_multi(s, nq).to(DEV)
    res = []
    for p32 in ("1", "0"):
        env_switch.setenv("FD_PREFILL_POOL32", p32)
        plan = check_multi(case, q, True, what=f"pool offsets p32={p32} {dtype} D={D} nq={nq}")
        assert plan["path"] == "prefill" and plan["heads_per_block"] == (64 if nq * 4 <= 64 else 128)
        dec = Decoder(q, case.k, case.v, scale=s.scale, page_table=case.page_table, seq_lens=case.seq_lens,
                      T=s.T, causal=True)
        out, lse = dec()
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("lens, grows", [([4096, 0, 5000, 700, 2048, 3333], True),   # ragged, one empty
                                         ([5000] * 6, True),                           # all at T
                                         ([5000, 1, 1, 1, 1, 1], False),               # one long, many short
                                         ([31, 32, 33, 0, 64, 65], False)])            # a tile or two
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
def test_query_tiled_device_chunk(lens, grows, dtype, D):
    # Ragged paged calls on the automatic split count let the order pass pick
    # the chunk from the lengths (about a whole number of rounds of the
    # resident workgroups, never below the plan's chunk); the query-tiled
    # kernel and the combine read it back.  Every query and head against the
    # oracle, causal and not, the workspace poisoned first; planned as if for
    # the device's CUs and for 4 CUs, where the first two length sets get a
    # chunk above the plan's.
    s = inputs.spec("paged_ragged_bf16", B=len(lens), Hq=8, Hkv=2, T=5000, page_size=16, dtype=dtype, D=D)
    npages = [-(-n // s.page_size) for n in lens]
    num_pages = max(1, sum(npages))
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    table = torch.zeros((s.B, -(-s.T // s.page_size)), dtype=torch.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    host = inputs.Case(s, inputs.make_q(s), inputs.make_pool(s, num_pages, inputs._K),
                       inputs.make_pool(s, num_pages, inputs._V), table, torch.tensor(lens, dtype=torch.int32))
    case = host.to(DEV)
    q = inputs.make_q_multi(s, 16)
    for causal in (True, False):
        ref_out, ref_lse = oracle_mod.default().decode_multi(q, host.k, host.v, s.scale, causal=causal,
                                                             page_table=host.page_table, seq_lens=host.seq_lens)
        for cus in (0, 4):
            dec = Decoder(q.to(DEV), case.k, case.v, scale=s.scale, page_table=case.page_table,
                          seq_lens=case.seq_lens, T=s.T, causal=causal, num_cus=cus)
            plan = dec.plan
            assert plan["path"] == "prefill" and plan["head_blocks"] == 1 and plan["n_splits"] > 1
            dec.workspace.fill_(0xFF)
            what = f"device chunk {dtype} D={D} lens={lens} causal={causal} cus={cus}"
            parity.announce(f"{what} plan={plan}")
            out, lse = dec()
            torch.cuda.synchronize()
            parity.compare(host, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                           parity.max_abs_v(host), what)
            # the chunk the order pass chose: the first word of the
            # workspace's last 256 bytes
            chunk = int(dec.workspace[-256:-252].cpu().view(torch.int32)[0])
            assert chunk % 32 == 0 and chunk >= plan["chunk"] and chunk * plan["n_splits"] >= s.T, (chunk, plan)
            if cus == 4:
                assert (chunk > plan["chunk"]) == grows, (chunk, plan)
            # fd_split then fd_combine: the combine reads the chunk the split's
            # order pass left in the workspace; bit for bit fd_decode's result
            out_a, lse_a = out.clone(), lse.clone()
            dec.out.fill_(float("nan"))
            dec.lse.fill_(float("nan"))
            dec.split()
            dec.combine()
            torch.cuda.synchronize()
            assert torch.equal(out_a, dec.out) and torch.equal(lse_a, dec.lse)


@pytest.mark.parametrize("B", [1024, 1025])
def test_query_tiled_order_batch_limit(B):
    # The column order pass takes at most 1024 sequences: B=1024 runs its
    # columns longest first with the chunk chosen on the device, B=1025 in
    # the plain order.  Planned as for 512 CUs, so the KV axis splits; the
    # workspace poisoned first.  Every query of a sample of sequences (first,
    # last, shortest, longest and 12 seeded others) against the oracle
    s = inputs.spec("paged_ragged_bf16", B=B, Hq=4, Hkv=1, T=2048, page_size=16, len_lo=0, len_hi=2048)
    case = inputs.make_case(s, device=DEV)
    q = inputs.make_q_multi(s, 16, device=DEV)
    dec = Decoder(q, case.k, case.v, scale=s.scale, page_table=case.page_table, seq_lens=case.seq_lens,
                  T=s.T, causal=True, num_cus=512)
    plan = dec.plan
    assert plan["path"] == "prefill" and plan["head_blocks"] == 1 and plan["n_splits"] > 1
    dec.workspace.fill_(0xFF)
    parity.announce(f"order batch limit B={B} plan={plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    lens = case.lengths()
    g = torch.Generator().manual_seed(B)
    bs = {0, B - 1, min(range(B), key=lambda b: lens[b]), max(range(B), key=lambda b: lens[b])}
    bs |= set(torch.randint(0, B, (12,), generator=g).tolist())
    parity.all_queries(case, q, out.cpu().double().numpy(), lse.cpu().double().numpy(), sorted(bs), True,
                       f"order batch limit B={B}")
