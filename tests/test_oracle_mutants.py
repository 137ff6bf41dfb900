"""Plant one plausible mistake at a time in a copy of the oracle's C source and check
that at least one pin in ``oracle_pins`` catches it.  The real oracle is untouched:
each mutant is compiled into a temporary directory."""
import os

import pytest

import oracle
import oracle_pins

with open(oracle.SOURCE) as _f:
    _SRC = _f.read()

# (name, exact snippet of the oracle source, replacement)
MUTANTS = [
    ("decay_dropped", "row[j] *= a;", "row[j] *= 1.0;"),
    ("decay_sign", "const double a = exp(g[i]);", "const double a = exp(-g[i]);"),
    ("decay_on_columns", "for (int64_t j = 0; j < dv; ++j) row[j] *= a;",
     "for (int64_t j = 0; j < dv; ++j) row[j] *= exp(g[j % dk]);"),
    ("erase_sign", "row[j] -= bk * kp[j];", "row[j] += bk * kp[j];"),
    ("erase_without_beta", "row[j] -= bk * kp[j];", "row[j] -= k[i] * kp[j];"),
    ("erase_uses_q", "kp[j] += k[i] * row[j];", "kp[j] += q[i] * row[j];"),
    ("write_without_beta", "row[j] += bk * v[j];", "row[j] += k[i] * v[j];"),
    ("read_before_write", "o[j] += q[i] * row[j];", "o[j] += q[i] * (row[j] - beta * k[i] * v[j]);"),
    ("read_with_k", "o[j] += q[i] * row[j];", "o[j] += k[i] * row[j];"),
    ("init_ignored", "if (job->init) memcpy", "if (0) memcpy"),
    ("state_not_reset", "else memset(S, 0,", "else if (s == 0) memset(S, 0,"),
    ("head_index", "const int64_t r = t * H + h;", "const int64_t r = t * H + (h + 1) % H;"),
    ("last_token_skipped", "t < job->cu[s + 1]; ++t", "t + 1 < job->cu[s + 1]; ++t"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    assert _SRC.count(old) >= 1, f"snippet for {name} not found in the oracle source"
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(_SRC.replace(old, new, 1))
    lib = oracle.build(str(src), str(tmp_path / f"mutant_{name}.so"), extra_flags=("-w",))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
