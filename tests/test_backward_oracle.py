"""The oracle's reverse mode against its pins, and planted mistakes in copies of its
source that the pins must catch."""
import pytest

import backward_pins
import oracle

with open(oracle.SOURCE) as _f:
    _SRC = _f.read()


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", backward_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_backward_pin(orc, pin):
    pin(orc)


# (name, exact snippet of the reverse-mode source, replacement)
MUTANTS = [
    ("read_adjoint_missing", "A[i * dv + j] += qt[i] * dot[j];", "A[i * dv + j] += 0.0 * dot[j];"),
    ("dq_from_previous_state", "acc += Sn[i * dv + j] * dot[j];", "acc += Sp[i * dv + j] * dot[j];"),
    ("dv_without_beta", "dvv[r * dv + j] = bt * e[j];", "dvv[r * dv + j] = e[j];"),
    ("dbeta_erase_dropped", "for (int64_t j = 0; j < dv; ++j) db -= e[j] * u[j];", "(void)0;"),
    ("dk_erase_term_sign", "- bt * P[i * dv + j] * e[j];", "+ bt * P[i * dv + j] * e[j];"),
    ("dP_without_erase", "const double dp = A[i * dv + j] - bt * kt[i] * e[j];",
     "const double dp = A[i * dv + j];"),
    ("adjoint_not_decayed", "A[i * dv + j] = a * dp;", "A[i * dv + j] = dp;"),
    ("dg_on_undecayed_state", "acc += dp * P[i * dv + j];", "acc += dp * Sp[i * dv + j];"),
    ("dfinal_ignored", "if (dfinal) memcpy(A,", "if (0) memcpy(A,"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_backward_mistake_is_caught(tmp_path, name, old, new):
    assert _SRC.count(old) == 1, f"snippet for {name} not found exactly once in the oracle source"
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(_SRC.replace(old, new, 1))
    lib = oracle.build(str(src), str(tmp_path / f"mutant_{name}.so"), extra_flags=("-w",))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in backward_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
