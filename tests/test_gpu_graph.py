"""Decode calls captured into a HIP graph and replayed: the in-launch merge's
arrival counters are left in a state that only depends on the launch's own
arguments, so every replay of a captured fused or stream-mode call counts its
workgroups from zero and merges.  Each replay gets a new q (copied in by
eager work between replays) and is compared with the fp64 oracle; the
workspace starts full of foreign bytes.  An eager call after the replays
must find the counters usable too.  Query-tiled calls are captured the same
way: the order pass (whose split size follows the lengths written between
replays) and the V conversion passes (whose exponent follows V) run inside
the graph."""
from dataclasses import replace

import pytest
import torch

from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(kind):
    if kind == "fused":
        s = inputs.spec("mha32k_f16", Hq=16, Hkv=16, T=9000)
    elif kind == "fused_gqa":
        s = inputs.spec("gqa128k_bf16", B=2, T=7000)
    else:
        s = inputs.spec("paged_ragged_bf16", B=6, Hq=8, Hkv=2, T=6000, len_lo=0, len_hi=6000)
    case = inputs.make_case(s, device="cpu")
    if kind == "stream":
        case.seq_lens[2] = 0
    return case


def _decoder(kind, case):
    c = case.to(DEV)
    if kind == "stream":
        return Decoder(c.q, c.k, c.v, scale=case.spec.scale, page_table=c.page_table,
                       seq_lens=c.seq_lens, T=case.spec.T)
    n = 8 if kind == "fused" else 12
    return Decoder(c.q, c.k, c.v, scale=case.spec.scale, n_splits=n, fused_merge=True)


def _check(kind, case, dec, q_host, what):
    from oracle import oracle as oracle_mod
    c = case.to("cpu")
    ref_out, ref_lse = oracle_mod.default().decode(q_host, c.k, c.v, case.spec.scale,
                                                   page_table=c.page_table, seq_lens=c.seq_lens)
    parity.compare(case, dec.out.cpu().double().numpy(), dec.lse.cpu().double().numpy(),
                   ref_out, ref_lse, parity.max_abs_v(case), what)


@pytest.mark.parametrize("kind", ["fused", "fused_gqa", "stream"])
def test_graph_replays_of_fused_calls(kind):
    case = _case(kind)
    dec = _decoder(kind, case)
    assert dec.plan["fused"] and dec.plan["n_splits"] > 1
    assert dec.plan["stream"] == (kind == "stream")
    q_dev = dec.inputs[0]
    parity.announce(f"graph {kind}: plan={dec.plan}")
    dec.workspace.fill_(0xFF)                  # foreign counters and NaN partials
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec()
    torch.cuda.synchronize()
    for rep in range(5):
        q_host = inputs.make_q(replace(case.spec, seed=case.spec.seed + 11 * rep + 1))
        q_dev.copy_(q_host.to(DEV))
        dec.out.fill_(float("nan"))            # a replay that skipped its merge would leave NaN
        torch.cuda.synchronize()
        parity.announce(f"graph {kind}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        _check(kind, case, dec, q_host, f"graph {kind} replay {rep}")
    # eager calls on the same workspace after the replays, then one more replay
    for rep in range(2):
        q_host = inputs.make_q(replace(case.spec, seed=case.spec.seed + 97 + rep))
        q_dev.copy_(q_host.to(DEV))
        dec.out.fill_(float("nan"))
        parity.announce(f"graph {kind}: eager call {rep} after the replays")
        dec()
        torch.cuda.synchronize()
        _check(kind, case, dec, q_host, f"graph {kind} eager {rep}")
    dec.out.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    _check(kind, case, dec, q_host, f"graph {kind} replay after eager calls")
    del g


def test_graph_replays_of_split_and_combine():
    # a plan that merges with the combine kernel (the default for large
    # calls) captured as two launches: every replay with a new q matches the
    # oracle, and so does an eager call afterwards
    case = _case("fused_gqa")
    c = case.to(DEV)
    dec = Decoder(c.q, c.k, c.v, scale=case.spec.scale, n_splits=12, fused_merge=False)
    assert not dec.plan["fused"] and dec.plan["combine"] and dec.plan["n_splits"] > 1
    q_dev = dec.inputs[0]
    parity.announce(f"graph split+combine: plan={dec.plan}")
    dec.workspace.fill_(0xFF)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec()
    torch.cuda.synchronize()
    for rep in range(4):
        q_host = inputs.make_q(replace(case.spec, seed=case.spec.seed + 13 * rep + 5))
        q_dev.copy_(q_host.to(DEV))
        dec.out.fill_(float("nan"))
        torch.cuda.synchronize()
        parity.announce(f"graph split+combine: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        _check("fused_gqa", case, dec, q_host, f"graph split+combine replay {rep}")
    q_host = inputs.make_q(replace(case.spec, seed=case.spec.seed + 501))
    q_dev.copy_(q_host.to(DEV))
    dec.out.fill_(float("nan"))
    dec()
    torch.cuda.synchronize()
    _check("fused_gqa", case, dec, q_host, "graph split+combine eager after the replays")
    del g


def test_graph_replays_of_query_tiled_ordered_call():
    # a ragged paged call with 16 causal queries: the order pass, the
    # query-tiled kernel and the row combine captured once; between replays
    # eager work copies in new queries and new (shorter) lengths, so the
    # split size the order pass picks on the device changes from replay to
    # replay under the same host plan (planned as for 4 CUs, where it grows
    # past the planned chunk).  Every replay against the oracle.
    from oracle import oracle as oracle_mod
    s = inputs.spec("paged_ragged_bf16", B=6, Hq=8, Hkv=2, T=6000, len_lo=2000, len_hi=6000)
    case = inputs.make_case(s, device="cpu")
    c = case.to(DEV)
    nq = 16
    q_dev = inputs.make_q_multi(s, nq).to(DEV)
    dec = Decoder(q_dev, c.k, c.v, scale=s.scale, page_table=c.page_table, seq_lens=c.seq_lens, T=s.T,
                  causal=True, num_cus=4)
    plan = dec.plan
    assert plan["path"] == "prefill" and plan["head_blocks"] == 1 and plan["n_splits"] > 1
    lens_dev = dec.inputs[4]
    parity.announce(f"graph query-tiled ordered: plan={plan}")
    dec.workspace.fill_(0xFF)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec()
    torch.cuda.synchronize()
    full = case.seq_lens.clone()
    gen = torch.Generator().manual_seed(77)
    chunks = set()
    for rep in range(4):
        q_host = inputs.make_q_multi(replace(s, seed=s.seed + 7 * rep + 3), nq)
        # each sequence keeps between none and all of its cached tokens
        lens = (full.double() * torch.rand(s.B, generator=gen, dtype=torch.float64)).to(torch.int32)
        if rep == 0:
            lens = full.clone()
        q_dev.copy_(q_host.to(DEV))
        lens_dev.copy_(lens.to(DEV))
        dec.out.fill_(float("nan"))
        torch.cuda.synchronize()
        parity.announce(f"graph query-tiled ordered: replay {rep} lens={lens.tolist()}")
        g.replay()
        torch.cuda.synchronize()
        chunks.add(int(dec.workspace[-256:-252].cpu().view(torch.int32)[0]))
        ref_out, ref_lse = oracle_mod.default().decode_multi(q_host, case.k, case.v, s.scale, causal=True,
                                                             page_table=case.page_table, seq_lens=lens)
        hc = replace(case, seq_lens=lens)
        parity.compare(hc, dec.out.cpu().double().numpy(), dec.lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(hc), f"graph query-tiled ordered replay {rep}")
    assert len(chunks) > 1, chunks
    del g


def test_graph_replays_of_converted_v_prefill():
    # bf16 prefill with 1024 query rows per kv head: the two V conversion
    # passes and the query-tiled kernel captured once.  Between replays eager
    # work writes a new V, scaled by a different power of two each time, so
    # the exponent the passes pick changes under the same graph; every
    # replay against the oracle.
    from oracle import oracle as oracle_mod
    s = inputs.spec("gqa128k_bf16", B=1, T=300)
    case = inputs.make_case(s, device="cpu")
    c = case.to(DEV)
    nq = 256
    q_host = inputs.make_q_multi(s, nq)
    q_dev = q_host.to(DEV)
    dec = Decoder(q_dev, c.k, c.v, scale=s.scale, causal=True)
    assert dec.plan["path"] == "prefill" and dec.plan["workspace_bytes"] > 0
    v_dev = dec.inputs[2]
    parity.announce(f"graph converted-V prefill: plan={dec.plan}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec()
    torch.cuda.synchronize()
    for rep, e in enumerate((0, 9, -13, 4)):
        v_host = (case.v.float() * 2.0 ** e).to(case.v.dtype)     # exact: a power of two
        qr = inputs.make_q_multi(replace(s, seed=s.seed + 5 * rep + 1), nq)
        v_dev.copy_(v_host.to(DEV))
        q_dev.copy_(qr.to(DEV))
        dec.out.fill_(float("nan"))
        torch.cuda.synchronize()
        parity.announce(f"graph converted-V prefill: replay {rep}, V x 2^{e}")
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle_mod.default().decode_multi(qr, case.k, v_host, s.scale, causal=True)
        hc = replace(case, v=v_host)
        parity.compare(hc, dec.out.cpu().double().numpy(), dec.lse.cpu().double().numpy(), ref_out, ref_lse,
                       parity.max_abs_v(hc), f"graph converted-V prefill replay {rep}")
    del g
