"""The seeded input generators (CPU): determinism, shapes and structure."""
import torch

from split_kv_fd_amd import inputs


def small(name, **kw):
    return inputs.spec(name, **kw)


def test_deterministic_and_shapes():
    s = small("gqa128k_bf16", B=2, T=512)
    a = inputs.make_case(s)
    b = inputs.make_case(s)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert a.q.shape == (2, 32, 128) and a.k.shape == (2, 8, 512, 128)
    assert a.k.dtype == torch.bfloat16
    assert s.G == 4


def test_sequence_redraw_matches_full_case():
    s = small("mha32k_f16", B=3, Hq=4, Hkv=4, T=256)
    c = inputs.make_case(s)
    k1, v1 = inputs.make_kv_seq(s, 1)
    assert torch.equal(c.k[1], k1) and torch.equal(c.v[1], v1)


def test_spiky_keys_are_exact_powers_of_two():
    s = small("gqa128k_bf16", B=1, T=1000)
    pos = inputs.spike_positions(s, 0)
    assert pos.numel() == 10 and len(set(pos.tolist())) == 10
    k, _ = inputs.make_kv_seq(s, 0)
    plain = inputs._randn((s.Hkv, s.T, s.D), s.dtype, "cpu", s.seed, inputs._K, 0)
    mask = torch.zeros(s.T, dtype=torch.bool)
    mask[pos] = True
    assert torch.equal(k[:, mask].float(), plain[:, mask].float() * 4)
    assert torch.equal(k[:, ~mask], plain[:, ~mask])


def test_hot_query_head():
    s = small("gqa_b64_bf16", B=4)
    q = inputs.make_q(s)
    plain = inputs._randn((s.B, s.Hq, s.D), s.dtype, "cpu", s.seed, inputs._Q)
    ratio = (q.float() / plain.float()).nan_to_num(1.0)
    hot = (ratio == 8).all(dim=-1)
    assert hot.sum(dim=1).tolist() == [1] * 4


def test_ragged_paged_layout():
    s = inputs.spec("paged_ragged_bf16")
    lens, table, num_pages = inputs.paged_layout(s)
    assert lens.shape == (16,) and lens.dtype == torch.int32
    assert int(lens.min()) >= 1024 - 1 and int(lens.max()) <= 65536
    assert bool((lens % 16 != 0).any())
    npg = [-(-int(n) // 16) for n in lens]
    assert num_pages == sum(npg)
    used = torch.cat([table[b, :n] for b, n in enumerate(npg)])
    assert sorted(used.tolist()) == list(range(num_pages))
    assert table.shape == (16, 4096)


def test_reduced_paged_case():
    s = inputs.spec("paged_ragged_bf16", B=3, T=200, len_lo=17, len_hi=200)
    c = inputs.make_case(s)
    assert c.k.shape == (c.meta["num_pages"], 8, 16, 128)
    assert c.page_table.shape == (3, 13)
    assert c.seq_lens.max() <= 200


def test_scale_is_fp32_value():
    s = inputs.spec("mha32k_f16")
    assert s.scale == float(torch.tensor(128 ** -0.5, dtype=torch.float32))
