"""Randomised pins of the oracle (no GPU): the exact rewrites the method rests
on, checked on inputs hypothesis draws rather than on fixed sizes.

* The chunkwise UT-transform form ("序列维度（下）", the chunk equations and the
  FlashKDA matrix form) equals the token recurrence for any length, chunk size,
  key/value width and decay scale, partial last chunks included.
* The segment law (systems page, eq. (17)): the state after a sequence equals
  the segment pairs (M, S~) applied in order, for any cut points.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
from oracle import brute, chunk_form


def _inputs(seed, T, d, g_scale):
    rng = np.random.default_rng(seed)

    def unit(n):
        x = rng.standard_normal((n, d))
        return x / np.linalg.norm(x, axis=1, keepdims=True)
    q, k = unit(T), unit(T)
    v = rng.standard_normal((T, d))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, d)))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((d, d)) * 0.3
    return q, k, v, g, beta, S0


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


SETTINGS = settings(max_examples=30, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(1, 150), C=st.sampled_from([4, 16, 32, 64]),
       d=st.sampled_from([8, 16, 32]), g_scale=st.sampled_from([0.01, 0.3, 1.0]))
def test_chunk_form_equals_recurrence_everywhere(seed, T, C, d, g_scale):
    q, k, v, g, beta, S0 = _inputs(seed, T, d, g_scale)
    o, S = oracle.recurrent(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                            S0[None, None])
    oc, Sc = chunk_form.run(q, k, v, g, beta, S0, C=C)
    assert _rel(oc, o[:, 0]) < 1e-10
    assert _rel(Sc, S[0, 0]) < 1e-10


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(2, 90), d=st.sampled_from([8, 16]),
       n_cuts=st.integers(1, 6), g_scale=st.sampled_from([0.01, 0.3]),
       data=st.data())
def test_segment_pairs_applied_in_order_give_the_serial_state(seed, T, d, n_cuts, g_scale,
                                                              data):
    q, k, v, g, beta, S0 = _inputs(seed, T, d, g_scale)
    inner = sorted(set(data.draw(st.lists(st.integers(1, T - 1), min_size=1,
                                          max_size=n_cuts))))
    cuts = [0] + inner + [T]
    _, S_serial = oracle.recurrent(q[:, None], k[:, None], v[:, None], g[:, None],
                                   beta[:, None], S0[None, None])
    S = S0.copy()
    for a, b in zip(cuts[:-1], cuts[1:]):
        S = brute.apply_pair(brute.segment_pair(k[a:b], v[a:b], g[a:b], beta[a:b]), S)
    assert _rel(S, S_serial[0, 0]) < 1e-10


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), d=st.sampled_from([8, 16]),
       lengths=st.lists(st.integers(0, 40), min_size=1, max_size=6))
def test_packed_documents_are_independent_runs(seed, d, lengths):
    """cu_seqlens packing: each document runs from its own initial state, as if
    alone; an empty document passes its initial state through (systems page,
    on document boundaries)."""
    T = sum(lengths)
    if T == 0:
        lengths = lengths + [1]
        T = 1
    q, k, v, g, beta, _ = _inputs(seed, T, d, 0.3)
    rng = np.random.default_rng(seed + 1)
    N = len(lengths)
    S0 = rng.standard_normal((N, 1, d, d)) * 0.3
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o, S = oracle.recurrent(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], S0,
                            cu_seqlens=cu)
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        if a == b:
            assert np.array_equal(S[n], S0[n])
            continue
        on, Sn = oracle.recurrent(q[a:b, None], k[a:b, None], v[a:b, None], g[a:b, None],
                                  beta[a:b, None], S0[n:n + 1])
        assert np.array_equal(o[a:b], on) and np.array_equal(S[n], Sn[0])
