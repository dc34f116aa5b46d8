"""Sequence sharding of the KV axis (the context-parallel layout a
multi-GPU deployment would use), emulated on one GPU: every shard of the
cache is decoded on its own, and the shards' (out, lse) pairs merge by
log-sum-exp into the whole-cache result -- exact by the same shift
invariance as the split merge (zenaique explainer, interview answer on
exactness).  A shard that holds none of a sequence's tokens gives out = 0,
lse = -inf and drops out of the merge."""
import numpy as np
import pytest
import torch

from split_kv_fd_amd import inputs
from split_kv_fd_amd.decode import Decoder
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("shards", [2, 3, 5])
@pytest.mark.parametrize("name", ["gqa128k_bf16", "mha32k_f16"])
def test_shards_merge_by_lse(name, shards):
    T = 3000
    s = inputs.spec(name, B=3, Hq=8, Hkv=2 if name == "gqa128k_bf16" else 8, T=T)
    case = inputs.make_case(s).to(DEV)
    lens = [T, 1000, 1]                        # later shards of the short sequences are empty
    case.seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    cuts = [round(i * T / shards) for i in range(shards + 1)]
    outs, lses = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        k = case.k[:, :, lo:hi].contiguous()
        v = case.v[:, :, lo:hi].contiguous()
        sl = torch.tensor([min(max(n - lo, 0), hi - lo) for n in lens], dtype=torch.int32, device=DEV)
        out, lse = Decoder(case.q, k, v, scale=s.scale, seq_lens=sl)()
        torch.cuda.synchronize()
        outs.append(out.double().cpu())
        lses.append(lse.double().cpu())
    lse_all = torch.stack(lses)                           # [shards, B, Hq]
    big = torch.logsumexp(lse_all, 0)
    w = torch.exp(lse_all - big)                          # 0 for empty shards
    merged = (w[..., None] * torch.stack(outs)).sum(0)
    ref_out, ref_lse = parity.oracle_full(case)
    parity.compare(case, merged.numpy(), big.numpy(), ref_out, ref_lse, parity.max_abs_v(case),
                   f"{name} in {shards} shards")
    # the emptiest shard of the 1-token sequence contributes exactly nothing
    assert torch.all(lse_all[-1, 2] == -np.inf) and torch.all(outs[-1][2] == 0)
