"""Each plausible mistake planted in a copy of the oracle source must fail at least one pin.

The copy is compiled to a temporary library on the CPU; the real oracle is untouched.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
import pins

MUTANTS = {
    "causal_strict": ("return j <= ip;", "return j < ip;"),
    "window_inclusive": ("(ip - j) < window", "(ip - j) <= window"),
    "global_inclusive": ("j < n_global", "j <= n_global"),
    "window_not_causal": ("return j <= ip && ((ip - j)", "return j <= ip + 1 && ((ip - j)"),
    "no_max_subtraction": ("e = exp(s[j] - m);", "e = exp(s[j]);"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "value_as_key": ("(double)krow[j][c];", "(double)vrow[j][c];"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "query_index": ("dot += (double)q[c]", "dot += (double)q[0]"),
    "no_normalise": ("out[c] /= l;", "out[c] /= (l + 1.0);"),
    "top_left_causal": ("i + (Nkv - Nq), mode", "i, mode"),
    "page_slot": ("(size_t)(j % page_size)", "(size_t)((j + 1) % page_size)"),
    "decode_head": ("* H + h) * d;", "* H + 0) * d;"),
    "max_ignores_first": ("if (s[j] > m)", "if (j > 0 && s[j] > m)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique"
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(before, after))
    lib = obuild.build(str(msrc), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
