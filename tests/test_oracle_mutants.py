"""Plant plausible mistakes in copies of the oracle and check the pins catch
each one (CPU only; the planted copies live in a temporary directory).

A pin set that lets a dropped term, a wrong sign or index, or a transposed
operand through would not be evidence that the oracle is right, so every
mutant below must fail at least one pin in tests/oracle_pins.py.
"""
import os
import shutil

import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "fd_oracle.c")

# (name, exact text in fd_oracle.c, replacement)
MUTANTS = [
    ("drop_scale", "s[t] = scale * dot;", "s[t] = dot;"),
    ("gqa_modulo_map", "j = h / group;", "j = h % Hkv;"),
    ("q_reads_kv_head", "qoff = ((size_t)b * Hq + h)", "qoff = ((size_t)b * Hq + j)"),
    ("k_transposed",
     "return (((size_t)b * Hkv + j) * (size_t)T + t) * (size_t)D;",
     "return (((size_t)b * Hkv + j) * (size_t)T) * (size_t)D + t;"),
    ("lse_without_max", "lse[i] = m + log(l);", "lse[i] = log(l);"),
    ("no_normalisation", "for (d = 0; d < D; ++d) o[d] /= l;", ""),
    ("exp_sign_flipped", "s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    ("unstable_no_shift", "s[t] = exp(s[t] - m);", "s[t] = exp(s[t]);"),
    ("values_read_from_k", "o[d] += s[t] * fdo_load(v, vr + d, dtype);",
     "o[d] += s[t] * fdo_load(k, vr + d, dtype);"),
    ("drop_last_token", "for (t = 0; t < Tb; ++t) {\n            size_t vr",
     "for (t = 0; t < Tb - 1; ++t) {\n            size_t vr"),
    ("ignore_seq_lens", "int Tb = seq_lens ? seq_lens[b] : T;", "int Tb = T;"),
    ("page_index_swapped",
     "int32_t page = page_table[(size_t)b * max_pages + t / page_size];\n        int row = t % page_size;",
     "int32_t page = page_table[(size_t)b * max_pages + t % page_size];\n        int row = t / page_size;"),
    ("page_head_order",
     "return (((size_t)page * Hkv + j) * (size_t)page_size + row) * (size_t)D;",
     "return (((size_t)page * page_size + row) * (size_t)Hkv + j) * (size_t)D;"),
    ("f16_exponent_bias", "expo - 25", "expo - 24"),
    ("f16_subnormal_scale", "ldexp((double)mant, -24)", "ldexp((double)mant, -25)"),
    ("bf16_shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("max_takes_min", "if (s[t] > m) m = s[t];", "if (s[t] < m) m = s[t];"),
]


def _build_mutant(tmpdir, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant {name}: pattern must occur once"
    src = os.path.join(tmpdir, f"mut_{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    lib = os.path.join(tmpdir, f"libmut_{name}.so")
    oracle_mod.build(src=src, out=lib)
    return oracle_mod.Oracle(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = _build_mutant(str(tmp_path), name, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    shutil.rmtree(str(tmp_path), ignore_errors=True)


# Mistakes planted in the oracle's append-then-decode step (oracle.py).
PY_SRC = oracle_mod.__file__
APPEND_MUTANTS = [
    ("append_not_attended", "grown = (sl + 1).astype(np.int32)", "grown = sl.astype(np.int32)"),
    ("append_values_from_k", "v_att[b, :, t] = vn[b]", "v_att[b, :, t] = kn[b]"),
    ("append_heads_reversed", "k_att[b, :, t] = kn[b]", "k_att[b, :, t] = kn[b, ::-1]"),
    ("append_store_next_slot", "                    ka[b, :, t] = kn[b]",
     "                    ka[b, :, min(t + 1, T - 1)] = kn[b]"),
    ("append_store_skipped", "                    va[b, :, t] = vn[b]\n", "\n"),
    ("append_paged_row", "ka[pt[b, col], :, t % P] = kn[b]", "ka[pt[b, col], :, (t + 1) % P] = kn[b]"),
    ("append_spare_row", "k_att[num_pages + i, :, t % P] = kn[b]",
     "k_att[num_pages + i, :, (t + 1) % P] = kn[b]"),
]


def _load_py_mutant(name, old, new):
    import types
    text = open(PY_SRC).read()
    assert text.count(old) == 1, f"mutant {name}: pattern must occur once"
    mod = types.ModuleType(f"oracle_mut_{name}")
    mod.__file__ = PY_SRC                      # same directory: the same C library
    exec(compile(text.replace(old, new), PY_SRC, "exec"), mod.__dict__)
    return mod.Oracle(oracle_mod.default().path)


@pytest.mark.parametrize("name,old,new", APPEND_MUTANTS, ids=[m[0] for m in APPEND_MUTANTS])
def test_append_mutant_is_caught(name, old, new):
    orc = _load_py_mutant(name, old, new)
    caught = []
    for pin in oracle_pins.APPEND_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every append pin"


# Mistakes planted in the oracle's several-queries decode (oracle.py).
MULTI_MUTANTS = [
    ("multi_causal_off_by_one", "li = np.maximum(lens - (nq - 1 - i), 0) if causal else lens",
     "li = np.maximum(lens - (nq - i), 0) if causal else lens"),
    ("multi_causal_reversed", "li = np.maximum(lens - (nq - 1 - i), 0) if causal else lens",
     "li = np.maximum(lens - i, 0) if causal else lens"),
    ("multi_causal_ignored", "li = np.maximum(lens - (nq - 1 - i), 0) if causal else lens", "li = lens"),
    ("multi_first_query_only", "o, l = self.decode(np.ascontiguousarray(qa[:, i]), k, v,",
     "o, l = self.decode(np.ascontiguousarray(qa[:, 0]), k, v,"),
]


@pytest.mark.parametrize("name,old,new", MULTI_MUTANTS, ids=[m[0] for m in MULTI_MUTANTS])
def test_multi_mutant_is_caught(name, old, new):
    orc = _load_py_mutant(name, old, new)
    caught = []
    for pin in oracle_pins.MULTI_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every several-queries pin"
