"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Every mutant below is a one-line change to a temporary copy of
oracle/mla_oracle.c (a dropped term, a wrong sign, index or base, a swapped
operand); the copy is compiled with gcc and the pins of oracle_pins.py are
run against it.  A mutant that passes every pin would mean the pins cannot
tell that mistake from the real oracle.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")

MUTANTS = {
    "scale_dropped": ("scores[t] = p->softmax_scale * dot;", "scores[t] = dot;"),
    "lse_base2": ("*lse = mx + log(Z);", "*lse = mx + log2(Z);"),
    "lse_without_max": ("*lse = mx + log(Z);", "*lse = log(Z);"),
    "value_from_rope_side": ("out[l] += w * row_elem(p, vrow, l);",
                             "out[l] += w * row_elem(p, vrow, l + (p->Dqk - p->Dv));"),
    "not_normalised": ("double w = exp(scores[t] - mx) / Z;", "double w = exp(scores[t] - mx);"),
    "dot_over_latent_only": ("for (int d = 0; d < p->Dqk; ++d)\n            dot +=",
                             "for (int d = 0; d < p->Dv; ++d)\n            dot +="),
    "page_off_by_one": ("int64_t page = t / p->page_size;", "int64_t page = (t + 1) / p->page_size;"),
    "row_ignores_page": ("int64_t row = t % p->page_size;", "int64_t row = 0;"),
    "fp8_scale_dropped": ("return e4m3_value[((const uint8_t *)row)[d]] * p->cache_scale;",
                          "return e4m3_value[((const uint8_t *)row)[d]];"),
    "fp8_subnormal_wrong": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "fp8_bias_wrong": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "bf16_shift_wrong": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "merge_weight_sign": ("double w = exp(ls[s] - total);", "double w = exp(total - ls[s]);"),
    "merge_lse_no_max": ("double total = mx + log(Z);", "double total = log(Z);"),
    "merge_empty_nan": ("if (mx == -INFINITY) {\n            lse[r] = -INFINITY;\n            continue;\n        }", ""),
    "span_start_ignored": ("const void *krow = token_row(p, b, t0 + t);",
                           "const void *krow = token_row(p, b, t);"),
    "value_row_of_wrong_token": ("const void *vrow = token_row(p, b, t0 + t);",
                                 "const void *vrow = token_row(p, b, t0 + (t + 1) % L);"),
    "max_not_tracked": ("if (scores[t] > mx)\n            mx = scores[t];", "mx = 0.0;"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    lib = oracle.load(oracle.build(path, os.path.join(workdir, f"lib{name}.so"),
                                   extra_flags=("-w",)))
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
