"""GPU parity of the fused append-KV decode step (fd_append_decode) against
the oracle's append-then-decode: out / lse within the decode tolerances, and
the caches after the call equal to the oracle's bit for bit (only the new
token's slot changes)."""
import pytest
import torch

from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def contiguous_case(name, lens, **kw):
    s = inputs.spec(name, B=len(lens), **kw)
    case = inputs.make_case(s).to(DEV)
    case.seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return case


def new_token(case, step=0):
    return inputs.make_new_token(case.spec, step, device="cpu")


def paged_case(s, lens):
    """A paged case whose table gives every sequence max_pages distinct pool
    pages (randomly placed), so no slot an append may write is shared."""
    max_pages = -(-s.T // s.page_size)
    n = s.B * max_pages
    g = torch.Generator().manual_seed(s.seed + 11)
    table = torch.randperm(n, generator=g).to(torch.int32).reshape(s.B, max_pages)
    case = inputs.Case(s, inputs.make_q(s), inputs.make_pool(s, n, 1), inputs.make_pool(s, n, 2),
                       table, torch.tensor(lens, dtype=torch.int32))
    return case.to(DEV)


@pytest.mark.parametrize("name,kw,path", [
    ("tiny_f32", dict(Hq=4, Hkv=4, T=300), "valu"),
    ("mha32k_f16", dict(Hq=8, Hkv=8, T=700), "valu"),
    ("mha32k_f16", dict(Hq=8, Hkv=2, T=700, dtype="bf16"), "valu"),
    ("gqa128k_bf16", dict(Hq=8, Hkv=2, T=700), "mfma"),
    ("gqa128k_bf16", dict(Hq=8, Hkv=2, T=700, dtype="f16"), "mfma"),
    ("gqa128k_bf16", dict(Hq=64, Hkv=2, T=700), "mfma"),       # one workgroup, two 16-row blocks
    ("gqa128k_bf16", dict(Hq=64, Hkv=2, T=700), "valu"),       # four head blocks
    ("gqa128k_bf16", dict(Hq=8, Hkv=2, T=700, D=64), "mfma"),
])
def test_append_contiguous(name, kw, path):
    # lengths: empty, one, a tile edge, the last free slot, a full cache
    T = kw["T"]
    for n in (0, 1, 3, 7):
        case = contiguous_case(name, [0, 1, 128, T - 1, T, T // 3], **kw)
        kn, vn = new_token(case, n)
        parity.check_append(case, kn.to(DEV), vn.to(DEV), n_splits=n, path=path,
                            what=f"append {name} {kw} n={n} {path}")


@pytest.mark.parametrize("fused", [False, True])
def test_append_fused_and_combine_kernel(fused):
    case = contiguous_case("gqa128k_bf16", [5000, 17, 4096, 1], Hq=16, Hkv=4, T=5000)
    kn, vn = new_token(case)
    _, plan = parity.check_append(case, kn.to(DEV), vn.to(DEV), n_splits=9, fused_merge=fused,
                                  what=f"append fused={fused}")
    assert plan["fused"] == fused


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("P", [1, 16, 256])
def test_append_paged(path, P):
    # stream plans (automatic) and split grids; lengths ending inside a page,
    # on a page boundary (the new token opens the next page), and a full table
    s = inputs.spec("paged_ragged_bf16", B=5, Hq=8, Hkv=2, T=1024, page_size=P)
    lens = [0, 3 * P if 3 * P < 1024 else 512, 1024, 999, 1]
    for n in (0, 1, 5):
        case = paged_case(s, lens)
        kn, vn = new_token(case, n)
        _, plan = parity.check_append(case, kn.to(DEV), vn.to(DEV), n_splits=n, path=path,
                                      what=f"append paged P={P} n={n} {path}")
        assert plan["stream"] == (n == 0)


@pytest.mark.parametrize("G,dtype", [(32, "bf16"), (24, "f16")])
def test_append_paged_two_row_blocks(G, dtype):
    # 17..32 query heads per kv head: the split kernel's two row blocks (value
    # product over V transposed through LDS) in stream mode and on a split
    # grid, with the appended token folded in as the last step
    s = inputs.spec("paged_ragged_bf16", B=4, Hq=G * 2, Hkv=2, T=1024, page_size=16, dtype=dtype)
    lens = [0, 48, 1024, 700]
    for n in (0, 5):
        case = paged_case(s, lens)
        kn, vn = new_token(case, n)
        _, plan = parity.check_append(case, kn.to(DEV), vn.to(DEV), n_splits=n, path="mfma",
                                      what=f"append paged two blocks G={G} {dtype} n={n}")
        assert plan["heads_per_block"] == 32 and plan["stream"] == (n == 0)


def test_append_successive_steps():
    # a decode loop: each step appends one token and the caller advances the
    # lengths; the cache the GPU builds step by step stays equal to the
    # oracle's, and every step's output matches
    s = inputs.spec("paged_ragged_bf16", B=3, Hq=8, Hkv=2, T=512)
    case = paged_case(s, [30, 47, 0])
    for step in range(5):
        kn, vn = new_token(case, step)
        parity.check_append(case, kn.to(DEV), vn.to(DEV), what=f"append step {step}")
        case.seq_lens += 1


def test_append_matches_decode_of_stored_cache():
    # After the append, a plain decode over the grown lengths reads the
    # stored rows from the cache: it must agree with the append's result.
    case = contiguous_case("gqa128k_bf16", [100, 2000, 0], Hq=16, Hkv=4, T=2048)
    kn, vn = new_token(case)
    app = Decoder(case.q, case.k, case.v, scale=case.spec.scale, seq_lens=case.seq_lens,
                  k_new=kn.to(DEV), v_new=vn.to(DEV))
    parity.announce("append then decode of the stored cache")
    out_a, lse_a = (x.clone() for x in app())
    grown = case.seq_lens + 1
    dec = Decoder(case.q, case.k, case.v, scale=case.spec.scale, seq_lens=grown)
    out_d, lse_d = dec()
    torch.cuda.synchronize()
    assert torch.allclose(out_a, out_d, rtol=0, atol=2e-6) and torch.allclose(lse_a, lse_d, rtol=0, atol=2e-6)
