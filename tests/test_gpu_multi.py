"""GPU parity of decode with several queries per sequence (q [B, n_q, Hq,
D]), causal or not, against the oracle's per-query decode."""
import pytest
import torch

from oracle import oracle as oracle_mod
from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def check_multi(case, q, causal, n_splits=0, path=None, fused_merge=None, what=""):
    host = case.to("cpu")
    ref_out, ref_lse = oracle_mod.default().decode_multi(
        q.cpu(), host.k, host.v, case.spec.scale, causal=causal, page_table=host.page_table,
        seq_lens=host.seq_lens if host.seq_lens is not None else None)
    dec = Decoder(q, case.k, case.v, scale=case.spec.scale, page_table=case.page_table,
                  seq_lens=case.seq_lens, T=case.spec.T if case.page_table is not None else None,
                  n_splits=n_splits, path=path, fused_merge=fused_merge, causal=causal)
    if dec.workspace is not None:
        dec.workspace.fill_(0xFF)
    parity.announce(f"multi-query {what} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    if path in ("valu", "mfma"):
        assert dec.plan["path"] == path
    assert out.shape == q.shape[:3] + (case.spec.D,) and lse.shape == q.shape[:3]
    parity.compare(case, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse,
                   parity.max_abs_v(host), what)
    return dec.plan


def contiguous(name, lens, **kw):
    s = inputs.spec(name, B=len(lens), **kw)
    case = inputs.make_case(s).to(DEV)
    case.seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return case


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [2, 3, 8])
@pytest.mark.parametrize("G,dtype,path", [(1, "f32", "valu"), (1, "f16", "valu"), (4, "bf16", "mfma"),
                                          (4, "bf16", "valu"), (8, "f16", "mfma"), (2, "bf16", "mfma")])
def test_multi_contiguous(causal, nq, G, dtype, path):
    Hkv = 2
    case = contiguous("mha32k_f16", [700, 0, 1, 2, 129, 333], Hq=G * Hkv, Hkv=Hkv, T=700, dtype=dtype)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    for n in (0, 1, 5):
        check_multi(case, q, causal, n_splits=n, path=path,
                    what=f"G={G} nq={nq} causal={causal} {dtype} {path} n={n}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_multi_paged(causal, path):
    for P in (16, 256):
        s = inputs.spec("paged_ragged_bf16", B=5, Hq=8, Hkv=2, T=1500, page_size=P, len_lo=0, len_hi=1500)
        case = inputs.make_case(s).to(DEV)
        case.seq_lens[1] = 2
        q = inputs.make_q_multi(s, 4).to(DEV)
        for n in (0, 3):
            plan = check_multi(case, q, causal, n_splits=n, path=path,
                               what=f"paged P={P} causal={causal} {path} n={n}")
            assert plan["stream"] == (n == 0)


@pytest.mark.parametrize("fused", [False, True])
def test_multi_merges(fused):
    case = contiguous("gqa128k_bf16", [3000, 2500, 7], Hq=16, Hkv=4, T=3000)
    q = inputs.make_q_multi(case.spec, 4).to(DEV)
    plan = check_multi(case, q, True, n_splits=12, fused_merge=fused, what=f"merges fused={fused}")
    assert plan["fused"] == fused


def test_multi_d64_and_many_rows():
    # 8 queries x G = 8: 64 query rows per kv head -- two 32-row workgroups
    # on the matrix-core split kernel when forced, the query-tiled kernel
    # (one K/V read for all 64 rows) by default
    case = contiguous("gqa128k_bf16", [900, 64, 3], Hq=16, Hkv=2, T=900, D=64)
    q = inputs.make_q_multi(case.spec, 8).to(DEV)
    for causal in (False, True):
        plan = check_multi(case, q, causal, path="mfma", what=f"D=64 64 rows mfma causal={causal}")
        assert plan["head_blocks"] == 2 and plan["heads_per_block"] == 32
        plan = check_multi(case, q, causal, what=f"D=64 64 rows causal={causal}")
        assert plan["path"] == "prefill"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,G", [(3, 8), (4, 8), (5, 4), (8, 4)])
def test_multi_32_row_blocks(causal, nq, G):
    # 17..32 query rows per kv head: one workgroup, two matrix-core row
    # blocks on one K / V read; contiguous splits and paged stream mode
    Hkv = 2
    case = contiguous("gqa128k_bf16", [1500, 0, 2, 700], Hq=G * Hkv, Hkv=Hkv, T=1500)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    for n in (0, 1, 6):
        plan = check_multi(case, q, causal, n_splits=n, path="mfma",
                           what=f"32-row nq={nq} G={G} causal={causal} n={n}")
        assert plan["heads_per_block"] == 32
    s = inputs.spec("paged_ragged_bf16", B=4, Hq=G * Hkv, Hkv=Hkv, T=1500, len_lo=0, len_hi=1500)
    pcase = inputs.make_case(s).to(DEV)
    q = inputs.make_q_multi(s, nq).to(DEV)
    plan = check_multi(pcase, q, causal, path="mfma", what=f"32-row paged nq={nq} G={G} causal={causal}")
    assert plan["stream"] and plan["heads_per_block"] == 32


def test_multi_query_equals_single_query_decodes():
    # without the mask, each query's result is the one-query decode of it
    case = contiguous("gqa128k_bf16", [2000, 1000], Hq=8, Hkv=2, T=2000)
    q = inputs.make_q_multi(case.spec, 3).to(DEV)
    multi = Decoder(q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens, n_splits=4)
    out_m, lse_m = (x.clone() for x in multi())
    for i in range(3):
        single = Decoder(q[:, i].contiguous(), case.k, case.v, scale=case.spec.scale,
                         seq_lens=case.seq_lens, n_splits=4)
        out_s, lse_s = single()
        torch.cuda.synchronize()
        assert torch.allclose(out_m[:, i], out_s, rtol=0, atol=2e-6)
        assert torch.allclose(lse_m[:, i], lse_s, rtol=0, atol=2e-6)


@pytest.mark.parametrize("nq,G,dtype", [(1, 17, "bf16"), (3, 8, "f16"), (8, 4, "bf16"), (5, 4, "f16"), (1, 32, "f16")])
def test_rows_17_to_32_take_two_row_blocks(nq, G, dtype):
    # 17..32 query rows per kv head: the automatic plan takes the matrix-core
    # split kernel with two 16-row blocks (value product on 16x16x32 MFMAs
    # over V transposed through LDS), contiguous and paged, both masks
    case = contiguous("gqa128k_bf16", [3000, 1500, 0], Hq=G * 2, Hkv=2, T=3000, dtype=dtype)
    q = inputs.make_q_multi(case.spec, nq).to(DEV)
    for causal in ((False, True) if nq > 1 else (False,)):
        plan = check_multi(case, q, causal, what=f"two row blocks nq={nq} G={G} {dtype} causal={causal}")
        assert plan["path"] == "mfma" and plan["heads_per_block"] == 32 and plan["head_blocks"] == 1
    s = inputs.spec("paged_ragged_bf16", B=3, Hq=G * 2, Hkv=2, T=2500, page_size=16, len_lo=0, len_hi=2500,
                    dtype=dtype)
    pcase = inputs.make_case(s).to(DEV)
    pq = inputs.make_q_multi(s, nq).to(DEV)
    plan = check_multi(pcase, pq, nq > 1, what=f"two row blocks paged nq={nq} G={G} {dtype}")
    assert plan["path"] == "mfma" and plan["stream"] and plan["heads_per_block"] == 32


# ------------------------------------------------------------------ full-size workloads, every query of sampled sequences

@pytest.mark.parametrize("name,nq", [("gqa_b64_bf16", 8), ("gqa128k_bf16", 16), ("paged_ragged_bf16", 16)])
def test_full_size_many_rows(name, nq):
    # the workloads at full size with nq causal queries per sequence: 64
    # query rows per kv head, the query-tiled kernel with KV splits, as the
    # benchmark runs them; every query and head of the first, the last and
    # two random sequences against the oracle
    s = inputs.spec(name)
    case = inputs.make_case(s, device=DEV)
    q = inputs.make_q_multi(s, nq, device=DEV)
    dec = Decoder(q, case.k, case.v, scale=s.scale, page_table=case.page_table, seq_lens=case.seq_lens,
                  T=s.T if case.page_table is not None else None, causal=True)
    assert dec.plan["path"] == "prefill"
    parity.announce(f"full size {name} nq={nq} plan={dec.plan}")
    out, lse = dec()
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(s.seed + 11)
    bs = sorted(set([0, s.B - 1] + torch.randint(0, s.B, (2,), generator=g).tolist()))
    parity.all_queries(case, q, out.cpu().double().numpy(), lse.cpu().double().numpy(), bs, True,
                       f"full {name} nq={nq}")
    del dec, out, lse, q, case
    torch.cuda.empty_cache()
