"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle.c with one plausible mistake (a dropped term,
a wrong sign or index, a swapped operand, a wrong mask), compiled to its own
library; at least one pin must fail on it.  This shows the pins constrain the
oracle, rather than restating it.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j] = P->scale * acc;", "s[j] = acc;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no_max_shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "no_normalise": ("for (int64_t j = 0; j < n; ++j) s[j] /= l;", ""),
    "sum_counts_keys": ("l += s[j];", "l += 1.0;"),
    "causal_off_by_one": ("if (last + 1 < n) n = last + 1;", "if (last < n) n = last;"),
    "causal_top_left": ("int64_t last = (int64_t)i + len - P->Sq;", "int64_t last = (int64_t)i;"),
    "kv_lens_ignored": ("len = P->kv_lens[b];", "len = P->Skv;"),
    "gqa_modulo_map": ("const int g = h / (P->Hq / P->Hkv);", "const int g = h % P->Hkv;"),
    "v_reads_k": ("o[c] += p * elem(P->v, P->dt, voff + c);",
                  "o[c] += p * elem(P->k, P->dt, voff + c);"),
    "k_transposed": ("elem(P->k, P->dt, koff + c)",
                     "elem(P->k, P->dt, kvbase * d + ((int64_t)c * n + j) % (P->Skv * (int64_t)d))"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "empty_row_sees_first_key": ("if (n < 0) n = 0;", "if (n < 1) n = 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in oracle.c"
    mut = tmp_path / f"oracle_{name}.c"
    mut.write_text(src.replace(old, new, 1))
    so = oracle_build.build(str(tmp_path / f"lib_{name}.so"), str(mut), quiet=True)
    lib = oracle.load(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
