"""Pins for the fp64 oracle: checks against facts that do not come from it.

Each pin takes an `Oracle` and raises AssertionError when the oracle disagrees
with something fixed by the pages or by mathematics: closed forms, special
cases, library routines (torch's fp64 scaled_dot_product_attention, numpy's
float16 conversion), a 50-digit mpmath brute force, and invariants of the
exact softmax.  The same pins are run against deliberately broken builds of
the oracle (tests/test_oracle_mutants.py) to show each plausible mistake is
caught by at least one of them.

Sources for the facts pinned here:
  * "Kernel visualization: Flash Decoding" (tinyvolt): one query row per
    (batch, head); the split and combine listings (scale applied before the
    max; one division at the end).
  * Zenaique explainer, "What decode looks like" (shapes, GQA head counts)
    and its interview answer (split/combine equals the whole softmax by
    shift invariance).
  * dupenodi guide, "Walking through it" (exact result; paged/ragged KV and
    GQA grouping as variants).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if not np.all(np.isfinite(a) == np.isfinite(b)):
        raise AssertionError(f"{what}: finiteness differs")
    fin = np.isfinite(b)
    if np.any(a[~fin] != b[~fin]):
        raise AssertionError(f"{what}: infinities differ")
    err = float(np.max(np.abs(a[fin] - b[fin]), initial=0.0))
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _ints(rng, shape, lo=-3, hi=3):
    """Small integers: every dot product of these is exact in fp64."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


# ---------------------------------------------------------------- special cases

def pin_single_token(orc):
    """T = 1: the softmax has one weight equal to 1, so out = V[0] exactly and
    lse = the single logit (exact here: integer operands, power-of-two scale)."""
    rng = _rng(1)
    B, Hq, Hkv, D = 2, 4, 2, 8
    q = _ints(rng, (B, Hq, D))
    k = _ints(rng, (B, Hkv, 1, D))
    v = rng.standard_normal((B, Hkv, 1, D))
    scale = 0.25
    out, lse = orc.decode(q, k, v, scale)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h], v[b, h // G, 0]), "T=1 must return V[0]"
            s0 = scale * float(np.dot(q[b, h], k[b, h // G, 0]))
            assert lse[b, h] == s0, f"T=1 lse {lse[b, h]} != logit {s0}"


def pin_constant_values(orc):
    """V[t] = c for every t: the weights sum to one, so out = c."""
    rng = _rng(2)
    B, Hq, Hkv, T, D = 1, 2, 1, 300, 16
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D)) * 3
    c = rng.standard_normal(D)
    v = np.broadcast_to(c, (B, Hkv, T, D)).copy()
    out, _ = orc.decode(q, k, v, 0.3)
    _close(out, np.broadcast_to(c, out.shape), 1e-14, "constant V")


def pin_uniform_weights(orc):
    """q = 0 (or scale = 0): every logit is 0, out = mean_t V[t], lse = ln T."""
    rng = _rng(3)
    B, Hq, Hkv, T, D = 2, 4, 4, 123, 8
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    q0 = np.zeros((B, Hq, D))
    out, lse = orc.decode(q0, k, v, 0.7)
    _close(out, v.mean(axis=2), 1e-14, "q=0 mean")
    _close(lse, np.full((B, Hq), math.log(T)), 1e-14, "q=0 lse")
    out2, lse2 = orc.decode(rng.standard_normal((B, Hq, D)), k, v, 0.0)
    _close(out2, v.mean(axis=2), 1e-14, "scale=0 mean")
    _close(lse2, np.full((B, Hq), math.log(T)), 1e-14, "scale=0 lse")


def pin_two_tokens(orc):
    """T = 2: out = sigmoid(s0-s1) V0 + sigmoid(s1-s0) V1, lse = logaddexp(s0, s1)."""
    rng = _rng(4)
    B, Hq, Hkv, D = 3, 2, 1, 6
    q = _ints(rng, (B, Hq, D))
    k = _ints(rng, (B, Hkv, 2, D))
    v = rng.standard_normal((B, Hkv, 2, D))
    scale = 0.5
    out, lse = orc.decode(q, k, v, scale)
    for b in range(B):
        for h in range(Hq):
            s0 = scale * float(np.dot(q[b, h], k[b, 0, 0]))
            s1 = scale * float(np.dot(q[b, h], k[b, 0, 1]))
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            _close(out[b, h], w0 * v[b, 0, 0] + w1 * v[b, 0, 1], 1e-15, "two tokens")
            _close(lse[b, h], np.logaddexp(s0, s1), 1e-14, "two tokens lse")


def pin_dominant_logit(orc):
    """One key aligned with q so its logit exceeds every other by >= 60 (and,
    second case, by ~1000, past exp overflow): out = V[t*]."""
    rng = _rng(5)
    B, Hq, Hkv, T, D = 1, 2, 2, 200, 16
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    tstar = [17, 151]
    for gap in (60.0, 1000.0):
        kk = k.copy()
        for h in range(Hq):
            others = float(np.abs(k[0, h] @ q[0, h]).max())
            c = others + gap
            kk[0, h, tstar[h]] = q[0, h] * (c / float(q[0, h] @ q[0, h]))
        out, lse = orc.decode(q, kk, v, 1.0)
        for h in range(Hq):
            _close(out[0, h], v[0, h, tstar[h]], T * math.exp(-50), f"dominant (gap {gap})")
            s_star = float(kk[0, h, tstar[h]] @ q[0, h])
            _close(lse[0, h], s_star, 1e-12 * max(1.0, abs(s_star)), f"dominant lse (gap {gap})")


# ---------------------------------------------------------------- library routines

def pin_torch_sdpa(orc):
    """torch's fp64 scaled_dot_product_attention with enable_gqa (query heads
    map to kv heads in consecutive groups), and torch.logsumexp of the logits."""
    import torch
    rng = _rng(6)
    for (B, Hq, Hkv, T, D, scale) in [(2, 8, 2, 37, 16, 0.17), (1, 4, 4, 256, 64, 0.125),
                                      (2, 6, 3, 5, 8, 1.3)]:
        q = rng.standard_normal((B, Hq, D))
        k = rng.standard_normal((B, Hkv, T, D))
        v = rng.standard_normal((B, Hkv, T, D))
        out, lse = orc.decode(q, k, v, scale)
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[:, :, None, :], kt, vt, scale=scale, enable_gqa=(Hq != Hkv))[:, :, 0, :]
        _close(out, ref.numpy(), 1e-12, "torch sdpa")
        G = Hq // Hkv
        krep = kt.repeat_interleave(G, dim=1)
        logits = torch.matmul(krep, qt[..., None])[..., 0] * scale
        _close(lse, torch.logsumexp(logits, dim=-1).numpy(), 1e-12, "torch logsumexp")


def pin_mpmath_bruteforce(orc):
    """50-digit evaluation of the definition on tiny shapes."""
    import mpmath
    mpmath.mp.dps = 50
    rng = _rng(7)
    for (T, D) in [(1, 1), (3, 2), (8, 4), (5, 3)]:
        B, Hq, Hkv = 1, 2, 1
        q = rng.standard_normal((B, Hq, D)) * 2
        k = rng.standard_normal((B, Hkv, T, D)) * 2
        v = rng.standard_normal((B, Hkv, T, D))
        scale = 0.9
        out, lse = orc.decode(q, k, v, scale)
        for h in range(Hq):
            logits = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, h, d]) * mpmath.mpf(k[0, 0, t, d])
                                                     for d in range(D)) for t in range(T)]
            w = [mpmath.e ** s for s in logits]
            z = mpmath.fsum(w)
            for d in range(D):
                ref = mpmath.fsum(w[t] * mpmath.mpf(v[0, 0, t, d]) for t in range(T)) / z
                assert abs(out[0, h, d] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref))), "mpmath out"
            assert abs(lse[0, h] - float(mpmath.log(z))) <= 1e-14 * max(1.0, abs(float(mpmath.log(z)))), "mpmath lse"


def pin_f16_decoder(orc):
    """The oracle's binary16 decoder equals numpy's float16 -> float64 on all
    65536 bit patterns (NaN patterns map to NaN)."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.decode_f16_bits(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 decoder"


def pin_bf16_decoder(orc):
    """The oracle's bfloat16 decoder equals torch's bfloat16 -> float64."""
    import torch
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.decode_bf16_bits(int(b)) for b in bits.numpy().view(np.uint16)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decoder"


def pin_storage_dtypes(orc):
    """Reading f32 / f16 / bf16 storage gives the same result as handing the
    oracle the exactly-widened values in fp64 (decoding must be exact)."""
    import torch
    rng = _rng(8)
    B, Hq, Hkv, T, D = 1, 4, 2, 77, 16
    base = [rng.standard_normal(s).astype(np.float32) for s in
            ((B, Hq, D), (B, Hkv, T, D), (B, Hkv, T, D))]
    for tdt in (torch.float32, torch.float16, torch.bfloat16):
        q, k, v = (torch.from_numpy(x).to(tdt) for x in base)
        out, lse = orc.decode(q, k, v, 0.3)
        q64, k64, v64 = (x.to(torch.float64).numpy() for x in (q, k, v))
        out64, lse64 = orc.decode(q64, k64, v64, 0.3)
        assert np.array_equal(out, out64) and np.array_equal(lse, lse64), f"dtype {tdt}"


# ---------------------------------------------------------------- the method's exactness

def split_combine_model(q, k, v, scale, n_splits, tile):
    """The split method in fp64 (tinyvolt walkthrough): each split runs an
    online softmax over its tiles, keeping an unnormalised accumulator with
    its running max and sum; the combine aligns every split to the global
    max and divides once.  Written from the math, independent of the oracle.
    q [D]; k, v [T, D].  Returns (out [D], lse)."""
    T = k.shape[0]
    size = -(-T // n_splits)
    parts = []
    for s in range(n_splits):
        lo, hi = s * size, min(T, (s + 1) * size)
        m, l, acc = -math.inf, 0.0, np.zeros(k.shape[1])
        for j in range(lo, hi, tile):
            z = scale * (k[j:min(hi, j + tile)] @ q)
            m_new = max(m, float(z.max()))
            a = math.exp(m - m_new) if m > -math.inf else 0.0
            p = np.exp(z - m_new)
            l = a * l + float(p.sum())
            acc = a * acc + p @ v[j:min(hi, j + tile)]
            m = m_new
        parts.append((m, l, acc))
    mg = max(m for m, _, _ in parts)
    lg = sum(math.exp(m - mg) * l for m, l, _ in parts if l > 0)
    og = sum(math.exp(m - mg) * a for m, l, a in parts if l > 0)
    return og / lg, mg + math.log(lg)


def pin_split_invariance(orc):
    """The split-and-merge result equals the whole softmax for every split
    count, including counts that do not divide T and empty splits."""
    rng = _rng(9)
    T, D = 997, 32
    q = rng.standard_normal((1, 1, D)) * 2
    k = rng.standard_normal((1, 1, T, D))
    v = rng.standard_normal((1, 1, T, D))
    k[0, 0, ::97] *= 4  # a few spiky keys
    out, lse = orc.decode(q, k, v, 1 / 8)
    for n in (1, 2, 3, 7, 8, 32, 128, 997):
        for tile in (1, 16, 64):
            o2, l2 = split_combine_model(q[0, 0], k[0, 0], v[0, 0], 1 / 8, n, tile)
            _close(out[0, 0], o2, 1e-12, f"split model n={n} tile={tile}")
            _close(lse[0, 0], l2, 1e-12, f"split model lse n={n}")


# ---------------------------------------------------------------- invariants

def pin_token_permutation(orc):
    """Permuting the cached tokens (K and V together) leaves the result."""
    rng = _rng(10)
    B, Hq, Hkv, T, D = 2, 4, 2, 150, 16
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    perm = rng.permutation(T)
    o1, l1 = orc.decode(q, k, v, 0.4)
    o2, l2 = orc.decode(q, k[:, :, perm], v[:, :, perm], 0.4)
    _close(o1, o2, 1e-13, "token permutation")
    _close(l1, l2, 1e-13, "token permutation lse")


def pin_gqa_equals_repeated_mha(orc):
    """GQA equals MHA with every kv head repeated for its group of query heads."""
    rng = _rng(11)
    B, Hq, Hkv, T, D = 2, 12, 3, 64, 8
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    o1, l1 = orc.decode(q, k, v, 0.35)
    G = Hq // Hkv
    o2, l2 = orc.decode(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.35)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "GQA vs repeated MHA"


def pin_paged_equals_contiguous(orc):
    """A paged pool read through a shuffled page table equals the contiguous
    cache gathered from it; ragged lengths cut each sequence (incl. lengths
    that end inside a page)."""
    rng = _rng(12)
    B, Hq, Hkv, D = 3, 4, 2, 8
    for P in (1, 4, 16):
        lens = np.array([5 * P + 3 if P > 1 else 9, 2 * P, 1], np.int32)
        maxp = int(-(-lens.max() // P)) + 1
        T = maxp * P
        npg = [-(-int(n) // P) for n in lens]
        num_pages = sum(npg) + 2
        perm = rng.permutation(num_pages)
        table = np.zeros((B, maxp), np.int32)
        off = 0
        for b in range(B):
            table[b, :npg[b]] = perm[off:off + npg[b]]
            off += npg[b]
        kp = rng.standard_normal((num_pages, Hkv, P, D))
        vp = rng.standard_normal((num_pages, Hkv, P, D))
        q = rng.standard_normal((B, Hq, D))
        out, lse = orc.decode(q, kp, vp, 0.5, page_table=table, seq_lens=lens)
        for b in range(B):
            n = int(lens[b])
            t = np.arange(n)
            kc = kp[table[b, t // P], :, t % P, :].transpose(1, 0, 2)[None]
            vc = vp[table[b, t // P], :, t % P, :].transpose(1, 0, 2)[None]
            o2, l2 = orc.decode(q[b:b + 1], kc, vc, 0.5)
            assert np.array_equal(out[b], o2[0]), f"paged vs contiguous P={P} b={b}"
            assert np.array_equal(lse[b], l2[0]), f"paged lse P={P} b={b}"


def pin_ragged_lengths(orc):
    """seq_lens[b] = n reads exactly the first n tokens: huge values stored
    past n change nothing; n = 0 gives out = 0, lse = -inf (our convention)."""
    rng = _rng(13)
    B, Hq, Hkv, T, D = 3, 2, 1, 40, 8
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    lens = np.array([17, 40, 0], np.int32)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, lens[b]:] = 1e6
        v2[b, :, lens[b]:] = -1e6
    out, lse = orc.decode(q, k2, v2, 0.5, seq_lens=lens)
    for b in range(2):
        n = int(lens[b])
        o2, l2 = orc.decode(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.5)
        assert np.array_equal(out[b], o2[0]) and np.array_equal(lse[b], l2[0]), f"ragged b={b}"
    assert np.all(out[2] == 0.0) and np.all(lse[2] == -np.inf), "empty sequence convention"


def pin_convexity_bounds(orc):
    """out is a convex combination of value rows and max_t s_t <= lse <=
    max_t s_t + ln T."""
    rng = _rng(14)
    B, Hq, Hkv, T, D = 2, 4, 4, 333, 16
    q = rng.standard_normal((B, Hq, D)) * 3
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    out, lse = orc.decode(q, k, v, 0.25)
    vmin, vmax = v.min(axis=2), v.max(axis=2)
    assert np.all(out >= vmin - 1e-12) and np.all(out <= vmax + 1e-12), "convex hull"
    smax = 0.25 * np.einsum("bhd,bhtd->bht", q, k).max(axis=2)
    assert np.all(lse >= smax - 1e-12) and np.all(lse <= smax + math.log(T) + 1e-12), "lse bounds"


def pin_linearity_in_values(orc):
    """out(a V + b V') = a out(V) + b out(V') for fixed q, K."""
    rng = _rng(15)
    B, Hq, Hkv, T, D = 1, 4, 2, 90, 8
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v1 = rng.standard_normal((B, Hkv, T, D))
    v2 = rng.standard_normal((B, Hkv, T, D))
    o1, _ = orc.decode(q, k, v1, 0.5)
    o2, _ = orc.decode(q, k, v2, 0.5)
    o3, _ = orc.decode(q, k, 2.5 * v1 - 0.75 * v2, 0.5)
    _close(o3, 2.5 * o1 - 0.75 * o2, 1e-13, "linearity in V")


def pin_row_subset(orc):
    """Computing a subset of (b, h) rows gives exactly those rows of the full result."""
    rng = _rng(16)
    B, Hq, Hkv, T, D = 3, 4, 2, 50, 8
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    full, lse = orc.decode(q, k, v, 0.5)
    rows = [11, 0, 5, 6]
    sub, lsub = orc.decode(q, k, v, 0.5, rows=rows)
    for i, r in enumerate(rows):
        assert np.array_equal(sub[i], full[r // Hq, r % Hq]), "row subset"
        assert lsub[i] == lse[r // Hq, r % Hq], "row subset lse"


# ---------------------------------------------------------------- golden fixtures

def load_golden():
    cases = []
    for name in sorted(os.listdir(GOLDEN_DIR)):
        if name.endswith(".json"):
            with open(os.path.join(GOLDEN_DIR, name)) as f:
                cases.append((name, json.load(f)))
    return cases


def pin_golden_fixtures(orc):
    """Hand-derived worked examples stored under tests/golden/."""
    cases = load_golden()
    assert cases, "no golden fixtures found"
    for name, c in cases:
        q = np.array(c["q"], np.float64)
        k = np.array(c["k"], np.float64)
        v = np.array(c["v"], np.float64)
        kw = {}
        if "page_table" in c:
            kw["page_table"] = np.array(c["page_table"], np.int32)
        if "seq_lens" in c:
            kw["seq_lens"] = np.array(c["seq_lens"], np.int32)
        out, lse = orc.decode(q, k, v, float(c["scale"]), **kw)
        exp_out = np.array([[[float(x) for x in row] for row in hb] for hb in c["expected_out"]])
        exp_lse = np.array([[float(x) for x in hb] for hb in c["expected_lse"]])
        _close(out, exp_out, c["tol"], f"golden {name}")
        _close(lse, exp_lse, c["tol"], f"golden {name} lse")


# ---------------------------------------------------------------- append, then decode

def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


def pin_append_to_empty(orc):
    """T_b = 0: after the append the sequence is the new token alone, so out
    = v_new exactly and lse = its logit (exact: integer operands); the cache
    changes at token 0 only."""
    rng = _rng(41)
    B, Hq, Hkv, T, D = 2, 4, 2, 5, 8
    q = _ints(rng, (B, Hq, D))
    kn = _ints(rng, (B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    out, lse, ka, va = orc.append_decode(q, kn, vn, k, v, 0.5, np.zeros(B, np.int32))
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h], vn[b, h // G]), "append to empty: out != v_new"
            assert lse[b, h] == 0.5 * float(np.dot(q[b, h], kn[b, h // G])), "append to empty: lse"
    assert np.array_equal(ka[:, :, 0], kn) and np.array_equal(va[:, :, 0], vn), "append: token 0 not stored"
    assert np.array_equal(ka[:, :, 1:], k[:, :, 1:]) and np.array_equal(va[:, :, 1:], v[:, :, 1:]), \
        "append: other tokens changed"


def pin_append_two_tokens(orc):
    """T_b = 1: two tokens, so out = sigma(s0 - s1) V0 + sigma(s1 - s0) v_new
    and lse = s1 + log(1 + exp(s0 - s1)) (logistic closed form)."""
    rng = _rng(42)
    B, Hq, Hkv, T, D = 1, 3, 1, 4, 6
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    kn = rng.standard_normal((B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    scale = 0.7
    out, lse, _, _ = orc.append_decode(q, kn, vn, k, v, scale, np.ones(B, np.int32))
    for h in range(Hq):
        s0 = scale * float(np.dot(q[0, h], k[0, 0, 0]))
        s1 = scale * float(np.dot(q[0, h], kn[0, 0]))
        ref = _sigmoid(s0 - s1) * v[0, 0, 0] + _sigmoid(s1 - s0) * vn[0, 0]
        _close(out[0, h], ref, 1e-14, "append T_b=1 out")
        _close(lse[0, h], s1 + math.log1p(math.exp(s0 - s1)), 1e-14, "append T_b=1 lse")


def pin_append_mpmath(orc):
    """50-digit brute force over the cached tokens 0 .. T_b-1 and the new
    token, on ragged tiny cases, contiguous and paged with shuffled pages;
    the stored rows sit exactly at the new token's slot."""
    import mpmath
    mpmath.mp.dps = 50
    rng = _rng(43)
    B, Hq, Hkv, T, D, P = 3, 4, 2, 8, 3, 2
    G = Hq // Hkv
    q = rng.standard_normal((B, Hq, D)) * 2
    k = rng.standard_normal((B, Hkv, T, D)) * 2
    v = rng.standard_normal((B, Hkv, T, D))
    kn = rng.standard_normal((B, Hkv, D)) * 2
    vn = rng.standard_normal((B, Hkv, D))
    lens = np.array([3, 0, 7], np.int32)
    scale = 0.8
    # paged copy of the same caches: page i of sequence b is pool page perm[b*n + i]
    n = T // P
    perm = rng.permutation(B * n)
    table = perm.reshape(B, n).astype(np.int32)
    kp = np.zeros((B * n, Hkv, P, D))
    vp = np.zeros((B * n, Hkv, P, D))
    for b in range(B):
        for i in range(n):
            kp[table[b, i]] = k[b, :, i * P:(i + 1) * P]
            vp[table[b, i]] = v[b, :, i * P:(i + 1) * P]
    res_c = orc.append_decode(q, kn, vn, k, v, scale, lens)
    res_p = orc.append_decode(q, kn, vn, kp, vp, scale, lens, page_table=table)
    for out, lse, _, _ in (res_c, res_p):
        for b in range(B):
            for h in range(Hq):
                j = h // G
                keys = [k[b, j, t] for t in range(lens[b])] + [kn[b, j]]
                vals = [v[b, j, t] for t in range(lens[b])] + [vn[b, j]]
                logits = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, h, d]) * mpmath.mpf(x[d])
                                                         for d in range(D)) for x in keys]
                w = [mpmath.e ** s for s in logits]
                z = mpmath.fsum(w)
                for d in range(D):
                    ref = float(mpmath.fsum(w[t] * mpmath.mpf(vals[t][d]) for t in range(len(w))) / z)
                    assert abs(out[b, h, d] - ref) <= 1e-14 * max(1.0, abs(ref)), "append mpmath out"
                ref_l = float(mpmath.log(z))
                assert abs(lse[b, h] - ref_l) <= 1e-14 * max(1.0, abs(ref_l)), "append mpmath lse"
    _, _, kc, vc = res_c
    _, _, kpa, vpa = res_p
    for b in range(B):
        t = int(lens[b])
        assert np.array_equal(kc[b, :, t], kn[b]) and np.array_equal(vc[b, :, t], vn[b]), "contiguous slot"
        pg, row = table[b, t // P], t % P
        assert np.array_equal(kpa[pg, :, row], kn[b]) and np.array_equal(vpa[pg, :, row], vn[b]), "paged slot"
    assert int(np.sum(kc != k)) == B * Hkv * D and int(np.sum(vc != v)) == B * Hkv * D, "contiguous: one row per (b, j)"
    assert int(np.sum(kpa != kp)) == B * Hkv * D and int(np.sum(vpa != vp)) == B * Hkv * D, "paged: one row per (b, j)"


def pin_append_full_cache(orc):
    """A full cache (T_b = T, or every page of the table in use) has no slot:
    the new token is still attended and nothing is stored.  Checked against
    a decode over caches one token longer built by concatenation."""
    rng = _rng(44)
    B, Hq, Hkv, T, D, P = 2, 2, 1, 6, 4, 3
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    kn = rng.standard_normal((B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    lens = np.array([T, 2], np.int32)
    out, lse, ka, va = orc.append_decode(q, kn, vn, k, v, 1.1, lens)
    k2 = np.concatenate([k, kn[:, :, None]], axis=2)
    v2 = np.concatenate([v, vn[:, :, None]], axis=2)
    ref, ref_l = orc.decode(q[0:1], k2[0:1], v2[0:1], 1.1)
    _close(out[0:1], ref, 1e-15, "full cache out")
    _close(lse[0:1], ref_l, 1e-15, "full cache lse")
    assert np.array_equal(ka[0], k[0]) and np.array_equal(va[0], v[0]), "full cache must stay unchanged"
    # paged: a table of T / P pages all in use
    table = np.array([[1, 0], [3, 2]], np.int32)
    kp = np.zeros((4, Hkv, P, D))
    vp = np.zeros((4, Hkv, P, D))
    for b in range(B):
        for i in range(2):
            kp[table[b, i]] = k[b, :, i * P:(i + 1) * P]
            vp[table[b, i]] = v[b, :, i * P:(i + 1) * P]
    out_p, lse_p, kpa, vpa = orc.append_decode(q, kn, vn, kp, vp, 1.1, lens, page_table=table)
    _close(out_p, out, 1e-15, "full paged table == full contiguous cache")
    _close(lse_p, lse, 1e-15, "full paged table lse")
    assert np.array_equal(kpa[table[0]], kp[table[0]]), "full paged cache must stay unchanged"


APPEND_PINS = [pin_append_to_empty, pin_append_two_tokens, pin_append_mpmath, pin_append_full_cache]


# ---------------------------------------------------------------- several queries per sequence

def pin_multi_single_query_is_decode(orc):
    """n_q = 1 (causal or not) is the one-query decode; the library routine
    here is the same oracle's decode, checked on its own pins above."""
    rng = _rng(51)
    B, Hq, Hkv, T, D = 2, 4, 2, 40, 8
    q = rng.standard_normal((B, 1, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    lens = np.array([40, 7], np.int32)
    ref, ref_l = orc.decode(q[:, 0], k, v, 0.3, seq_lens=lens)
    for causal in (False, True):
        out, lse = orc.decode_multi(q, k, v, 0.3, causal=causal, seq_lens=lens)
        assert np.array_equal(out[:, 0], ref) and np.array_equal(lse[:, 0], ref_l), "n_q = 1"


def pin_multi_causal_first_query(orc):
    """Causal with n_q = T_b: query 0 sees token 0 alone, so its out = V[0]
    exactly and lse = its logit (integer operands); the last query sees all
    T_b tokens (the plain decode)."""
    rng = _rng(52)
    B, Hq, Hkv, D, T = 1, 2, 1, 4, 6
    q = _ints(rng, (B, T, Hq, D))
    k = _ints(rng, (B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    out, lse = orc.decode_multi(q, k, v, 0.5, causal=True)
    for h in range(Hq):
        assert np.array_equal(out[0, 0, h], v[0, 0, 0]), "causal query 0 must return V[0]"
        assert lse[0, 0, h] == 0.5 * float(np.dot(q[0, 0, h], k[0, 0, 0])), "causal query 0 lse"
    ref, ref_l = orc.decode(q[:, T - 1], k, v, 0.5)
    _close(out[:, T - 1], ref, 0.0, "causal last query == decode")
    _close(lse[:, T - 1], ref_l, 0.0, "causal last query lse")


def pin_multi_mpmath(orc):
    """50-digit brute force of every query's softmax, causal and not, on
    ragged contiguous and paged caches."""
    import mpmath
    mpmath.mp.dps = 50
    rng = _rng(53)
    B, nq, Hq, Hkv, T, D, P = 2, 3, 4, 2, 6, 3, 2
    G = Hq // Hkv
    q = rng.standard_normal((B, nq, Hq, D)) * 2
    k = rng.standard_normal((B, Hkv, T, D)) * 2
    v = rng.standard_normal((B, Hkv, T, D))
    lens = np.array([5, 2], np.int32)
    n = T // P
    table = rng.permutation(B * n).reshape(B, n).astype(np.int32)
    kp = np.zeros((B * n, Hkv, P, D))
    vp = np.zeros((B * n, Hkv, P, D))
    for b in range(B):
        for i in range(n):
            kp[table[b, i]] = k[b, :, i * P:(i + 1) * P]
            vp[table[b, i]] = v[b, :, i * P:(i + 1) * P]
    for causal in (False, True):
        results = [orc.decode_multi(q, k, v, 0.6, causal=causal, seq_lens=lens),
                   orc.decode_multi(q, kp, vp, 0.6, causal=causal, seq_lens=lens, page_table=table)]
        for out, lse in results:
            for b in range(B):
                for i in range(nq):
                    L = max(0, lens[b] - (nq - 1 - i)) if causal else lens[b]
                    for h in range(Hq):
                        j = h // G
                        if L == 0:
                            assert np.all(out[b, i, h] == 0) and np.isneginf(lse[b, i, h]), "empty query"
                            continue
                        logits = [mpmath.mpf(0.6) * mpmath.fsum(mpmath.mpf(q[b, i, h, d]) * mpmath.mpf(k[b, j, t, d])
                                                               for d in range(D)) for t in range(L)]
                        w = [mpmath.e ** x for x in logits]
                        z = mpmath.fsum(w)
                        for d in range(D):
                            ref = float(mpmath.fsum(w[t] * mpmath.mpf(v[b, j, t, d]) for t in range(L)) / z)
                            assert abs(out[b, i, h, d] - ref) <= 1e-14 * max(1.0, abs(ref)), "multi mpmath out"
                        ref_l = float(mpmath.log(z))
                        assert abs(lse[b, i, h] - ref_l) <= 1e-14 * max(1.0, abs(ref_l)), "multi mpmath lse"


def pin_multi_query_permutation(orc):
    """Without the causal mask the queries are independent: permuting them
    permutes the results (and equal queries give equal results)."""
    rng = _rng(54)
    B, nq, Hq, Hkv, T, D = 2, 4, 2, 1, 30, 8
    q = rng.standard_normal((B, nq, Hq, D))
    q[:, 3] = q[:, 1]
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    out, lse = orc.decode_multi(q, k, v, 0.4)
    perm = [2, 0, 3, 1]
    out_p, lse_p = orc.decode_multi(q[:, perm], k, v, 0.4)
    assert np.array_equal(out_p, out[:, perm]) and np.array_equal(lse_p, lse[:, perm]), "query permutation"
    assert np.array_equal(out[:, 3], out[:, 1]), "equal queries"


MULTI_PINS = [pin_multi_single_query_is_decode, pin_multi_causal_first_query, pin_multi_mpmath,
              pin_multi_query_permutation]


ALL_PINS = [
    pin_single_token, pin_constant_values, pin_uniform_weights, pin_two_tokens,
    pin_dominant_logit, pin_torch_sdpa, pin_mpmath_bruteforce, pin_f16_decoder,
    pin_bf16_decoder, pin_storage_dtypes, pin_split_invariance, pin_token_permutation,
    pin_gqa_equals_repeated_mha, pin_paged_equals_contiguous, pin_ragged_lengths,
    pin_convexity_bounds, pin_linearity_in_values, pin_row_subset, pin_golden_fixtures,
]
