"""Seeded synthetic inputs for single-query decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  The tests feed the same tensors to the HIP library and
(as host copies) to the CPU oracle; the benchmark uses it for its workloads.

Recipe (every draw is seeded; nothing is read from disk):
  * values ~ N(0, 1) drawn in fp32 with a torch.Generator on the requested
    device, rounded once to the storage dtype (round to nearest even);
  * one generator per tensor stream and per sequence, seeded from
    (config seed, stream id, sequence index), so one sequence of a large
    case can be redrawn alone;
  * structure is applied after rounding with power-of-two factors, which is
    exact: spiky keys (x4 on a random 1% of the positions of each sequence,
    all kv heads), a hot query head (x8 on one random head per sequence);
  * ragged lengths ~ U{lo .. hi} with at least one length not a multiple of
    the page size; pages are handed out from a random permutation of the
    pool, so consecutive pages of a sequence are scattered.

Layouts: q [B, Hq, D]; contiguous K/V [B, Hkv, T, D]; paged pools
[num_pages, Hkv, P, D] with page_table [B, max_pages] int32 (unused entries
0) and seq_lens [B] int32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Stream ids inside one config seed.
_Q, _K, _V, _AUX = 0, 1, 2, 3


@dataclass(frozen=True)
class Spec:
    """Shape and structure of one decode workload."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int                      # KV length (max length when ragged)
    dtype: str                  # "f32" | "f16" | "bf16"
    seed: int
    n_splits: int = 0           # 0: library's automatic choice
    spiky_k_frac: float = 0.0   # fraction of positions whose K rows are x4
    hot_q: bool = False         # one head per sequence has q x8
    paged: bool = False
    page_size: int = 16
    len_lo: int = 0             # ragged lengths ~ U{len_lo .. len_hi}
    len_hi: int = 0
    page_shuffle: bool = True   # hand out pool pages in random order

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        """1/sqrt(D) as the fp32 value handed to both sides."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))


# The five workloads: a tiny fp32 case, long-context MHA, long-context GQA
# with spiky keys, a paged ragged batch, and a high-batch GQA serving step.
SPECS = {
    "tiny_f32": Spec("tiny_f32", B=1, Hq=4, Hkv=4, D=64, T=1024, dtype="f32",
                     seed=100, n_splits=4),
    "mha32k_f16": Spec("mha32k_f16", B=1, Hq=32, Hkv=32, D=128, T=32768,
                       dtype="f16", seed=200),
    "gqa128k_bf16": Spec("gqa128k_bf16", B=4, Hq=32, Hkv=8, D=128, T=131072,
                         dtype="bf16", seed=300, spiky_k_frac=0.01),
    "paged_ragged_bf16": Spec("paged_ragged_bf16", B=16, Hq=32, Hkv=8, D=128,
                              T=65536, dtype="bf16", seed=400, paged=True,
                              page_size=16, len_lo=1024, len_hi=65536),
    "gqa_b64_bf16": Spec("gqa_b64_bf16", B=64, Hq=64, Hkv=8, D=128, T=32768,
                         dtype="bf16", seed=500, hot_q=True),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally resized (structure is kept)."""
    return replace(SPECS[name], **overrides)


@dataclass
class Case:
    spec: Spec
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    page_table: Optional[torch.Tensor] = None
    seq_lens: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def device(self):
        return self.q.device

    def to(self, device) -> "Case":
        mv = lambda x: None if x is None else x.to(device)
        return Case(self.spec, self.q.to(device), self.k.to(device), self.v.to(device),
                    mv(self.page_table), mv(self.seq_lens), dict(self.meta))

    def lengths(self) -> list:
        """Valid KV length of each sequence."""
        if self.seq_lens is None:
            return [self.spec.T] * self.spec.B
        return [int(x) for x in self.seq_lens.cpu().tolist()]


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    s = 0
    for part in key:
        s = (s * 1_000_003 + int(part)) % (2**62)
    g.manual_seed(s)
    return g


def _randn(shape, dtype: str, device, *key) -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(device, *key), device=device,
                    dtype=torch.float32)
    return x.to(DTYPES[dtype])


def make_q(s: Spec, device="cpu") -> torch.Tensor:
    q = _randn((s.B, s.Hq, s.D), s.dtype, device, s.seed, _Q)
    if s.hot_q:
        g = _gen("cpu", s.seed, _AUX, 1)
        heads = torch.randint(0, s.Hq, (s.B,), generator=g)
        for b in range(s.B):
            q[b, int(heads[b])] *= 8
    return q


def spike_positions(s: Spec, b: int) -> torch.Tensor:
    """Sorted positions of sequence b whose K rows are scaled by 4."""
    n = int(round(s.spiky_k_frac * s.T))
    g = _gen("cpu", s.seed, _AUX, 2, b)
    return torch.sort(torch.randperm(s.T, generator=g)[:n]).values


def make_kv_seq(s: Spec, b: int, device="cpu"):
    """K, V of one sequence of a contiguous case: each [Hkv, T, D]."""
    k = _randn((s.Hkv, s.T, s.D), s.dtype, device, s.seed, _K, b)
    v = _randn((s.Hkv, s.T, s.D), s.dtype, device, s.seed, _V, b)
    if s.spiky_k_frac > 0:
        pos = spike_positions(s, b).to(device)
        k[:, pos, :] *= 4
    return k, v


def ragged_lengths(s: Spec) -> torch.Tensor:
    g = _gen("cpu", s.seed, _AUX, 3)
    lens = torch.randint(s.len_lo, s.len_hi + 1, (s.B,), generator=g, dtype=torch.int64)
    if s.page_size > 1 and bool((lens % s.page_size == 0).all()):
        lens[0] = lens[0] + 1 if lens[0] < s.len_hi else lens[0] - 1
    return lens.to(torch.int32)


def paged_layout(s: Spec):
    """(seq_lens [B], page_table [B, max_pages], num_pages) of a paged case."""
    lens = ragged_lengths(s)
    P = s.page_size
    max_pages = -(-s.T // P)
    npages = [-(-int(n) // P) for n in lens]
    num_pages = sum(npages)
    perm = torch.randperm(num_pages, generator=_gen("cpu", s.seed, _AUX, 4)).to(torch.int32)
    if not s.page_shuffle:
        perm = torch.arange(num_pages, dtype=torch.int32)
    table = torch.zeros((s.B, max_pages), dtype=torch.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    return lens, table, num_pages


def make_pool(s: Spec, num_pages: int, which: int, device="cpu",
              pages_per_draw: int = 4096) -> torch.Tensor:
    """A K (which=1) or V (which=2) pool [num_pages, Hkv, P, D], drawn in blocks."""
    pool = torch.empty((num_pages, s.Hkv, s.page_size, s.D), dtype=DTYPES[s.dtype],
                       device=device)
    for i, p0 in enumerate(range(0, num_pages, pages_per_draw)):
        p1 = min(num_pages, p0 + pages_per_draw)
        pool[p0:p1] = _randn((p1 - p0, s.Hkv, s.page_size, s.D), s.dtype, device,
                             s.seed, which, i)
    return pool


def make_case(s: Spec, device="cpu") -> Case:
    """Draw every tensor of a workload on `device`."""
    q = make_q(s, device)
    if s.paged:
        lens, table, num_pages = paged_layout(s)
        k = make_pool(s, num_pages, _K, device)
        v = make_pool(s, num_pages, _V, device)
        return Case(s, q, k, v, table.to(device), lens.to(device),
                    {"num_pages": num_pages, "max_pages": table.shape[1]})
    k = torch.empty((s.B, s.Hkv, s.T, s.D), dtype=DTYPES[s.dtype], device=device)
    v = torch.empty_like(k)
    for b in range(s.B):
        k[b], v[b] = make_kv_seq(s, b, device)
    return Case(s, q, k, v)


def make_q_multi(s: Spec, n_queries: int, device="cpu") -> torch.Tensor:
    """Queries of several tokens per sequence: [B, n_queries, Hq, D]."""
    return _randn((s.B, n_queries, s.Hq, s.D), s.dtype, device, s.seed, _Q, 100 + n_queries)


def make_new_token(s: Spec, step: int = 0, device="cpu"):
    """K, V rows of one appended decode token per sequence: each [B, Hkv, D]
    (seeded by the config seed and the step index)."""
    k = _randn((s.B, s.Hkv, s.D), s.dtype, device, s.seed, _AUX, 5, step, 0)
    v = _randn((s.B, s.Hkv, s.D), s.dtype, device, s.seed, _AUX, 5, step, 1)
    return k, v


def describe(s: Spec) -> dict:
    """The recipe of a workload as plain values (for logs and results)."""
    d = {"name": s.name, "B": s.B, "Hq": s.Hq, "Hkv": s.Hkv, "G": s.G, "D": s.D,
         "T": s.T, "dtype": s.dtype, "seed": s.seed, "scale": s.scale,
         "n_splits": s.n_splits or "auto"}
    if s.spiky_k_frac:
        d["spiky_k"] = f"x4 on {s.spiky_k_frac:.0%} of positions"
    if s.hot_q:
        d["hot_q"] = "x8 on one head per sequence"
    if s.paged:
        d.update(page_size=s.page_size, lengths=f"U{{{s.len_lo}..{s.len_hi}}}")
    return d
