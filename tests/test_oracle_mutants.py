"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle.c (or of the row-block evaluation,
oracle/rowblock.py) with one plausible mistake (a dropped term, a wrong sign
or index, a swapped operand, a wrong mask), compiled to its own library or
loaded as its own module; at least one pin must fail on it.  This shows the
pins constrain both evaluations, rather than restating them.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
SRC_RB = os.path.join(os.path.dirname(oracle.__file__), "rowblock.py")

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
            break
    assert failed, f"no pin catches mutant {name}"


MUTANTS_ROWBLOCK = {
    "dropped_scale": ("S.mul_(scale)", "S.mul_(1.0)"),
    "exp_sign": ("S.sub_(m[:, None])", "S.sub_(m[:, None]).neg_()"),
    "no_max_shift": ("S.sub_(m[:, None])", "S.sub_(0.0)"),
    "no_normalise": ("S.div_(torch.where(live, l, torch.ones_like(l))[:, None])", "pass"),
    "sum_counts_keys": ("l = S.sum(dim=1)", "l = (S > 0).sum(dim=1).double()"),
    "causal_off_by_one": ("(i + (n - Sq) + 1)", "(i + (n - Sq))"),
    "causal_top_left": ("(i + (n - Sq) + 1)", "(i + 1)"),
    "kv_lens_ignored": ("return [min(max(n, 0), Skv) for n in lens]", "return [Skv] * B"),
    "gqa_modulo_map": ("g = h // G", "g = h % Hkv"),
    "v_reads_k": ("torch.matmul(S, V[:kmax])", "torch.matmul(S, K[:kmax])"),
    "keys_reversed": ("torch.matmul(Qb, K[:kmax].T)", "torch.matmul(Qb, K[:kmax].flip(0).T)"),
    "lse_without_max": ("m + torch.log(l)", "torch.log(l)"),
    "mask_adds_zero": ('float("-inf"))\n    # pass 2', '0.0)\n    # pass 2'),
    "empty_row_sees_keys": ("live = cnt > 0", "live = cnt >= 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS_ROWBLOCK))
def test_rowblock_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS_ROWBLOCK[name]
    src = open(SRC_RB).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in rowblock.py"
    path = tmp_path / f"rowblock_{name}.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location(f"rowblock_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, FloatingPointError, RuntimeError):
            failed.append(pin.__name__)
            break
    assert failed, f"no pin catches rowblock mutant {name}"
