"""The layer oracle (decay gate, ShortConv prologue, RMSNorm + output-gate epilogue)
against its pins, and planted mistakes in copies of its source that the pins must
catch."""
import importlib.util
import os

import pytest

import layer_pins
from oracle import layer

with open(layer.__file__) as _f:
    _SRC = _f.read()


@pytest.mark.parametrize("pin", layer_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_layer_oracle_pin(pin):
    pin(layer)


# (name, exact snippet of oracle/layer.py, replacement)
MUTANTS = [
    ("gmin_wrong", "G_MIN = -5.0", "G_MIN = -4.0"),
    ("gate_scale_not_exponentiated", "np.exp(A)[None, :, None] * z", "A[None, :, None] * z"),
    ("gate_sigmoid_sign", "return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    ("gate_head_axis", "np.exp(A)[None, :, None] * z", "np.exp(A[::-1])[None, :, None] * z"),
    ("conv_taps_reversed", "acc += w[:, :, j] * hist[3 + t - j]", "acc += w[:, :, 3 - j] * hist[3 + t - j]"),
    ("conv_no_swish", "y[bos + t] = swish(acc)", "y[bos + t] = acc"),
    ("conv_cache_order", "hist = np.concatenate([c_in[s].transpose(2, 0, 1), x[bos:eos]], axis=0)",
     "hist = np.concatenate([c_in[s].transpose(2, 0, 1)[::-1], x[bos:eos]], axis=0)"),
    ("conv_cache_dropped", "c_in = np.zeros((nseq, H, d, 3)) if cache is None else _f64(cache)",
     "c_in = np.zeros((nseq, H, d, 3))"),
    ("conv_cache_out_newest_first", "c_out[s] = hist[-3:].transpose(1, 2, 0)",
     "c_out[s] = hist[-3:][::-1].transpose(1, 2, 0)"),
    ("l2norm_over_heads", "np.sum(y * y, axis=-1, keepdims=True)", "np.sum(y * y, axis=-2, keepdims=True)"),
    ("norm_sum_not_mean", "np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    ("norm_gate_linear", "return sigmoid(u) * (o / rms) * w", "return u * (o / rms) * w"),
    ("norm_weight_dropped", "return sigmoid(u) * (o / rms) * w", "return sigmoid(u) * (o / rms)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_layer_mistake_is_caught(tmp_path, name, old, new):
    assert _SRC.count(old) >= 1, f"snippet for {name} not found in oracle/layer.py"
    path = tmp_path / f"layer_{name}.py"
    path.write_text(_SRC.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location(f"layer_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in layer_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
