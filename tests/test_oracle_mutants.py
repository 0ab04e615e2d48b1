"""The oracle pins have teeth: plausible mistakes planted in a copy of the C
oracle (on the CPU, in a temporary directory) must each fail at least one pin.

The mutants cover the slips the pins are meant to catch: a dropped decay, the
decay applied after the erase, the erase dropped or with its sign flipped,
beta misplaced, the output read before the update, a transposed output, the
previous token's decay, and two gate slips (sigmoid sign, A_h outside exp).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

with open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c"), encoding="utf-8") as _fh:
    SRC = _fh.read()

DECAY = "    /* decay first: S <- Diag(alpha_t) S */\n"
UBLK = "    /* u = beta (v - S^T k), against the decayed state */\n"
WRITE = "    /* erase-and-write: S <- S + k u^T */\n"
OUT = "    /* o_t = S_t^T q_t */\n"


def _blocks(src):
    i0, i1, i2, i3 = (src.index(m) for m in (DECAY, UBLK, WRITE, OUT))
    end = src.index("  }\n}\n", i3)
    return src[:i0], src[i0:i1], src[i1:i2], src[i2:i3], src[i3:end], src[end:]


def _reorder(order):
    def f(src):
        head, d, u, w, o, tail = _blocks(src)
        parts = {"d": d, "u": u, "w": w, "o": o}
        return head + "".join(parts[c] for c in order) + tail
    return f


def _replace(old, new):
    def f(src):
        assert old in src, old
        return src.replace(old, new)
    return f


MUTANTS = {
    "decay_dropped": _replace("for (int32_t j = 0; j < dv; ++j) Si[j] *= a;",
                              "for (int32_t j = 0; j < dv; ++j) Si[j] *= 1.0;"),
    "decay_after_erase": _reorder("uwdo"),
    "output_before_update": _reorder("duow"),
    "erase_dropped": _replace("u[j] = bt * (vt[j] - u[j]);", "u[j] = bt * vt[j];"),
    "erase_sign": _replace("u[j] = bt * (vt[j] - u[j]);", "u[j] = bt * (vt[j] + u[j]);"),
    "beta_on_erase_only": _replace("u[j] = bt * (vt[j] - u[j]);", "u[j] = vt[j] - bt * u[j];"),
    "output_transposed": _replace(
        "for (int32_t j = 0; j < dv; ++j) ot[j] += Si[j] * qi;",
        "for (int32_t j = 0; j < dv; ++j) ot[i < dv ? i : 0] += Si[j] * qt[j < dk ? j : 0];"),
    "previous_token_decay": _replace("const double *gt = g + row * dk;",
                                     "const double *gt = g + (t > t0 ? row - H : row) * dk;"),
    "gate_sigmoid_sign": _replace("gr[c] = g_min * (1.0 / (1.0 + exp(-x)));",
                                  "gr[c] = g_min * (1.0 / (1.0 + exp(x)));"),
    "gate_scale_outside_exp": _replace("const double scale = exp(A_log ? A_log[h] : 0.0);",
                                       "const double scale = 1.0 + (A_log ? A_log[h] : 0.0);"),
    "softplus_wrong_branch": _replace("log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    "softplus_no_floor_term": _replace("(x > 0.0 ? x : 0.0) + log1p", "log1p"),
    "softplus_sign": _replace("gr[c] = -scale * sp;", "gr[c] = scale * sp;"),
}

PIN_TESTS = [
    pins.test_gate_closed_forms,
    pins.test_softplus_gate_closed_forms,
    pins.test_reduces_to_linear_attention,
    pins.test_delta_rule_retrieval,
    pins.test_decay_only_closed_form,
    lambda m: pins.test_matches_explicit_transition_matrices(m, 16),
    lambda m: pins.test_chunk_form_equals_recurrence(m, 16, 200),
    pins.test_segment_pairs_compose_to_serial_state,
    lambda m: pins.test_decode_replay_equals_explicit_steps(m, "bounded"),
    lambda m: pins.test_decode_replay_equals_explicit_steps(m, "softplus"),
    lambda m: pins.test_decode_window_equals_explicit_steps(m, "bounded"),
    lambda m: pins.test_decode_window_equals_explicit_steps(m, "softplus"),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(tmp_path, name):
    src = MUTANTS[name](SRC)
    assert src != SRC
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(c), "-o",
                    str(so), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = None
    real_path = oracle._LIB_PATH
    try:
        oracle._LIB_PATH = str(so)
        oracle._SRC = str(c)
        oracle._load()
        failed = []
        for t in PIN_TESTS:
            try:
                t(oracle)
            except AssertionError:
                failed.append(getattr(t, "__name__", "lambda"))
        assert failed, f"mutant {name} passed every pin"
    finally:
        oracle._lib = saved
        oracle._LIB_PATH = real_path
        oracle._SRC = os.path.join(os.path.dirname(real_path), "kda_oracle.c")


# The raw-input preprocessing is NumPy code in oracle/__init__.py: mutate it by
# substituting the functions, and check that a pin fails each time.
RAW_PIN_TESTS = [pins.test_raw_inputs_scale_invariance, pins.test_raw_inputs_reduce_to_normalised,
                 pins.test_raw_inputs_retrieval]
RAW_MUTANTS = {
    "normalise_by_squared_norm": ("l2_normalize",
                                  lambda x: np.asarray(x, np.float64) /
                                  np.maximum(np.sum(np.asarray(x, np.float64) ** 2, -1, keepdims=True), 1e-300)),
    "no_normalisation": ("l2_normalize", lambda x: np.asarray(x, np.float64)),
    "sigmoid_sign": ("sigmoid", lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, np.float64)))),
    "beta_logit_unchanged": ("sigmoid", lambda x: np.asarray(x, np.float64)),
}


@pytest.mark.parametrize("name", sorted(RAW_MUTANTS))
def test_raw_mutant_fails_a_pin(name, monkeypatch):
    attr, bad = RAW_MUTANTS[name]
    monkeypatch.setattr(oracle, attr, bad)
    failed = []
    for t in RAW_PIN_TESTS:
        try:
            t(oracle)
        except AssertionError:
            failed.append(t.__name__)
    assert failed, f"mutant {name} passed every pin"
