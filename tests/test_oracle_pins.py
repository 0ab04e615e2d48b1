"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it relies on.  Together they are chosen so that a
plausible slip in the oracle -- a dropped term, a wrong sign, decay applied
after the erase, the output read before the update, a transposed state, a
wrong gate -- fails at least one of them.  No expected value here comes from
the GPU path.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

import kda_gen
from oracle import brute, chunk_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(rng, T, H, dk, dv, g_scale=1.0):
    q = _unit_rows(rng, T * H, dk).reshape(T, H, dk)
    k = _unit_rows(rng, T * H, dk).reshape(T, H, dk)
    v = rng.standard_normal((T, H, dv))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, dk)))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# Gate: equation (5), "序列维度（下）", section "K3 的改动：下界衰减"
# ---------------------------------------------------------------------------
def test_gate_closed_forms(oracle_mod):
    z = np.array([0.0, 50.0, -50.0, 1.0, -2.5], dtype=np.float64).reshape(5, 1, 1)
    g = oracle_mod.gate(z, np.zeros(1), -5.0)[:, 0, 0]
    assert g[0] == -2.5                            # sigmoid(0) = 1/2
    assert abs(g[1] - (-5.0)) < 1e-15              # z -> +inf saturates at g_min
    assert abs(g[2]) < 1e-20                       # z -> -inf gives no decay
    assert abs(g[3] - (-5.0 / (1.0 + math.exp(-1.0)))) < 1e-15
    # the per-head log scale multiplies z inside the sigmoid
    rng = _rng(0)
    zz = rng.standard_normal((7, 3, 16))
    A = np.array([0.0, 0.7, -1.3])
    lhs = oracle_mod.gate(zz, A, -5.0)
    rhs = oracle_mod.gate(zz * np.exp(A)[None, :, None], None, -5.0)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-14)
    assert np.all(lhs < 0) and np.all(lhs > -5.0)
    # g_min scales the whole map linearly
    assert np.allclose(oracle_mod.gate(zz, A, -2.0) * 2.5, lhs, rtol=0, atol=1e-14)


def test_softplus_gate_closed_forms(oracle_mod):
    """The unbounded Kimi Linear gate, g = -e^A softplus(z) ("序列维度（下）",
    section "K3 的改动：下界衰减"): softplus(0) = ln 2, softplus(z) -> z for large
    z (no floor), -> e^z for very negative z, softplus(z) - softplus(-z) = z, and
    e^A multiplies outside."""
    z = np.array([0.0, 40.0, -40.0, 1.0, -2.5, 700.0], dtype=np.float64).reshape(6, 1, 1)
    g = oracle_mod.gate_softplus(z, np.zeros(1))[:, 0, 0]
    assert abs(g[0] + math.log(2.0)) < 1e-15
    assert abs(g[1] + 40.0) < 1e-12                 # linear, no lower bound
    assert abs(g[2] + math.exp(-40.0)) < 1e-30       # tiny decay for very negative z
    assert abs(g[3] + math.log(1.0 + math.e)) < 1e-15
    assert abs(g[4] + math.log(1.0 + math.exp(-2.5))) < 1e-15
    assert abs(g[5] + 700.0) < 1e-9                  # no overflow where exp(z) would
    rng = _rng(1)
    zz = rng.standard_normal((9, 3, 16)) * 4.0
    gp = oracle_mod.gate_softplus(zz, None)
    gm = oracle_mod.gate_softplus(-zz, None)
    assert np.allclose(gm - gp, zz, rtol=0, atol=1e-12)  # sp(z) - sp(-z) = z
    A = np.array([0.0, 0.9, -1.4])
    assert np.allclose(oracle_mod.gate_softplus(zz, A), gp * np.exp(A)[None, :, None],
                       rtol=1e-15, atol=0)
    assert np.all(gp < 0)
    # gate_of picks the map the inputs name
    inp = kda_gen.make_prefill(3, 64, 2, "f32", gate="softplus")
    assert np.array_equal(oracle_mod.gate_of(inp, inp.z.f64()),
                          oracle_mod.gate_softplus(inp.z.f64(), inp.A_log))


def test_gate_range_matches_page_numbers(oracle_mod):
    with open(GOLDEN, encoding="utf-8") as fh:
        gold = json.load(fh)
    z = np.linspace(-30, 30, 2001).reshape(-1, 1, 1)
    alpha = np.exp(oracle_mod.gate(z, None, -5.0))
    lb = gold["alpha_lower_bound"]
    assert alpha.min() > math.exp(-5.0)
    assert abs(math.exp(-5.0) - lb["value"]) <= lb["rel_tol"] * lb["value"]
    # 16 steps above g_min span less than 5 x 16 = 80, and e^80 fits bf16
    assert 5 * 16 == gold["subtile_log_decay_span"]["value"]
    e80 = gold["exp80"]
    assert abs(math.exp(80) - e80["value"]) <= e80["rel_tol"] * e80["value"]
    bf16_max = float(kda_gen.bf16_bits_to_f32(np.array([0x7F7F], dtype=np.uint16))[0])
    assert abs(bf16_max - gold["bf16_max"]["value"]) <= 0.01 * gold["bf16_max"]["value"]
    assert math.exp(80) < bf16_max


# ---------------------------------------------------------------------------
# Recurrence, equation (1) of the systems page ("KDA 上下文并行")
# ---------------------------------------------------------------------------
def test_reduces_to_linear_attention(oracle_mod):
    """alpha = 1 and mutually orthogonal keys: the erase term vanishes, so KDA is
    causal linear attention with write weight beta (the SemiAnalysis page,
    section "线性注意力"; the systems page on LASP-style summed states)."""
    rng = _rng(1)
    T, H, d = 96, 2, 128
    Qo, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = np.stack([Qo[:T].copy(), Qo[T - 1::-1][:T].copy()], axis=1)  # orthonormal per head
    q = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    beta = rng.uniform(0.05, 1.0, size=(T, H))
    g = np.zeros((T, H, d))
    o, S = oracle_mod.recurrent(q, k, v, g, beta)
    for h in range(H):
        S_ref = sum(beta[t, h] * np.outer(k[t, h], v[t, h]) for t in range(T))
        assert _rel(S[0, h], S_ref) < 1e-13
        scores = q[:, h] @ k[:, h].T                      # [T, T]
        causal = np.tril(scores * beta[None, :, h])       # output reads S_t (diagonal kept)
        o_ref = causal @ v[:, h]
        assert _rel(o[:, h], o_ref) < 1e-13


def test_delta_rule_retrieval(oracle_mod):
    """beta = 1 and unit keys: after each step S_t^T k_t = v_t exactly, whatever
    the decay and the prior state (delta rule, SemiAnalysis page "DeltaNet").
    With q = k the output is therefore v."""
    rng = _rng(2)
    T, H, d = 40, 3, 128
    k = _unit_rows(rng, T * H, d).reshape(T, H, d)
    v = rng.standard_normal((T, H, d))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, d))))
    beta = np.ones((T, H))
    S0 = rng.standard_normal((1, H, d, d))
    o, _ = oracle_mod.recurrent(k, k, v, g, beta, S0)
    assert np.max(np.abs(o - v)) < 1e-11


def test_decay_only_closed_form(oracle_mod):
    """k = 0 (or beta = 0): no write and no erase, so S_t = Diag(prod alpha) S_0."""
    rng = _rng(3)
    T, H, dk, dv = 33, 2, 128, 64
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=0.05)
    S0 = rng.standard_normal((1, H, dk, dv))
    for variant in ("k0", "beta0"):
        kk = np.zeros_like(k) if variant == "k0" else k
        bb = beta if variant == "k0" else np.zeros_like(beta)
        o, S = oracle_mod.recurrent(q, kk, v, g, bb, S0)
        G = np.cumsum(g, axis=0)                     # [T, H, dk], inclusive
        for h in range(H):
            St = np.exp(G[:, h, :])[:, :, None] * S0[0, h][None]     # [T, dk, dv]
            o_ref = np.einsum("tij,ti->tj", St, q[:, h])
            assert _rel(o[:, h], o_ref) < 1e-13
            assert _rel(S[0, h], St[-1]) < 1e-13


@pytest.mark.parametrize("d", [16, 128])
def test_matches_explicit_transition_matrices(oracle_mod, d):
    """The delta form (decay, u, rank-1 write) equals eq. (1) built as explicit
    matrices M_t = (I - beta k k^T) Diag(alpha) (oracle/brute.py)."""
    rng = _rng(4 + d)
    T, H = 64, 2
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, d, g_scale=0.1)
    S0 = rng.standard_normal((1, H, d, d)) * 0.3
    o, S = oracle_mod.recurrent(q, k, v, g, beta, S0)
    for h in range(H):
        ob, Sb = brute.run(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h])
        assert _rel(o[:, h], ob) < 1e-12
        assert _rel(S[0, h], Sb) < 1e-12


@pytest.mark.parametrize("C,T", [(16, 200), (64, 200), (64, 64), (64, 1)])
def test_chunk_form_equals_recurrence(oracle_mod, C, T):
    """The chunkwise UT-transform form (pages: "序列维度（下）" eq. (3)-(4) and the
    FlashKDA matrix form) equals the token recurrence, including a partial chunk."""
    rng = _rng(5 + C + T)
    H, d = 2, 128
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, d, g_scale=0.3)
    S0 = rng.standard_normal((1, H, d, d)) * 0.1
    o, S = oracle_mod.recurrent(q, k, v, g, beta, S0)
    for h in range(H):
        oc, Sc = chunk_form.run(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h], C=C)
        assert _rel(o[:, h], oc) < 1e-12
        assert _rel(S[0, h], Sc) < 1e-12


# ---------------------------------------------------------------------------
# Segment law, equation (17) and its derivation (systems page)
# ---------------------------------------------------------------------------
def test_segment_pairs_compose_to_serial_state(oracle_mod):
    rng = _rng(6)
    T, d = 60, 32
    q, k, v, g, beta = _rand_inputs(rng, T, 1, d, d, g_scale=0.05)
    q, k, v, g, beta = q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    S0 = rng.standard_normal((d, d))
    _, S_serial = oracle_mod.recurrent(q[:, None], k[:, None], v[:, None], g[:, None],
                                       beta[:, None], S0[None, None])
    S_serial = S_serial[0, 0]
    cuts = [0, 17, 18, 41, T]                      # includes a one-token segment
    pairs = [brute.segment_pair(k[a:b], v[a:b], g[a:b], beta[a:b])
             for a, b in zip(cuts[:-1], cuts[1:])]
    # sequential scan S <- M_j S + S~_j
    S = S0.copy()
    for p in pairs:
        S = brute.apply_pair(p, S)
    assert _rel(S, S_serial) < 1e-12
    # the composed pair, in either bracketing, maps S0 to the same state
    left = brute.compose(pairs[3], brute.compose(pairs[2], brute.compose(pairs[1], pairs[0])))
    right = brute.compose(brute.compose(pairs[3], pairs[2]), brute.compose(pairs[1], pairs[0]))
    assert _rel(left[0], right[0]) < 1e-12 and _rel(left[1], right[1]) < 1e-12
    assert _rel(brute.apply_pair(left, S0), S_serial) < 1e-12
    # not commutative: swapping two segments changes the result
    swapped = brute.compose(pairs[0], pairs[1])
    fwd = brute.compose(pairs[1], pairs[0])
    assert _rel(swapped[1], fwd[1]) > 1e-3
    # each pair is what the oracle produces from a zero state and from S0
    a, b = cuts[1], cuts[3]
    M, St = brute.segment_pair(k[a:b], v[a:b], g[a:b], beta[a:b])
    _, Sz = oracle_mod.recurrent(q[a:b, None], k[a:b, None], v[a:b, None], g[a:b, None],
                                 beta[a:b, None])
    assert _rel(Sz[0, 0], St) < 1e-12
    _, Sx = oracle_mod.recurrent(q[a:b, None], k[a:b, None], v[a:b, None], g[a:b, None],
                                 beta[a:b, None], S0[None, None])
    assert _rel(Sx[0, 0], M @ S0 + St) < 1e-12


def test_linear_in_values_and_initial_state(oracle_mod):
    rng = _rng(7)
    T, H, d = 50, 2, 64
    q, k, v1, g, beta = _rand_inputs(rng, T, H, d, d)
    v2 = rng.standard_normal(v1.shape)
    S1 = rng.standard_normal((1, H, d, d))
    S2 = rng.standard_normal((1, H, d, d))
    a, b = 0.7, -1.9
    o1, F1 = oracle_mod.recurrent(q, k, v1, g, beta, S1)
    o2, F2 = oracle_mod.recurrent(q, k, v2, g, beta, S2)
    o3, F3 = oracle_mod.recurrent(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2)
    assert _rel(o3, a * o1 + b * o2) < 1e-12
    assert _rel(F3, a * F1 + b * F2) < 1e-12


def test_resume_equals_one_pass(oracle_mod):
    rng = _rng(8)
    T, H, d = 90, 2, 128
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, d, g_scale=0.1)
    S0 = rng.standard_normal((1, H, d, d)) * 0.1
    o, S = oracle_mod.recurrent(q, k, v, g, beta, S0)
    for cut in (1, 37, 64, 89):
        oa, Sa = oracle_mod.recurrent(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], S0)
        ob, Sb = oracle_mod.recurrent(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], Sa)
        assert np.array_equal(np.concatenate([oa, ob]), o)
        assert np.array_equal(Sb, S)


def test_packed_documents_are_independent(oracle_mod):
    rng = _rng(9)
    lens = [5, 0, 70, 1, 24]
    T, H, d = sum(lens), 2, 128
    q, k, v, g, beta = _rand_inputs(rng, T, H, d, d)
    cu = kda_gen.cu_from_lengths(lens)
    S0 = rng.standard_normal((len(lens), H, d, d)) * 0.05
    o, S = oracle_mod.recurrent(q, k, v, g, beta, S0, cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, Sn = oracle_mod.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], S0[n:n + 1])
        assert np.array_equal(o[s:e], on)
        assert np.array_equal(S[n], Sn[0])
    # an empty document passes its initial state through
    assert np.array_equal(S[1], S0[1])


@pytest.mark.parametrize("gate", ["bounded", "softplus"])
def test_decode_replay_equals_explicit_steps(oracle_mod, gate):
    """Replay of the accepted drafts plus the bonus token (systems page, decode)
    from the saved state equals eq. (1) stepped explicitly over the same tokens;
    the rejected drafts leave no trace (no rollback needed)."""
    inp = kda_gen.make_decode(11, N=6, H=2, W=4, dtype="bf16", d=128,
                              accepted=[0, 1, 2, 3, 4, 2], gate=gate)
    o, S = oracle_mod.decode(inp)
    gfun = oracle_mod.gate_softplus if gate == "softplus" else \
        (lambda z, A: oracle_mod.gate(z, A, inp.g_min))
    gate_h = lambda z: gfun(z[None, None, :], inp.A_log[None, h:h + 1])[0, 0]
    for n in range(inp.N):
        a = int(inp.accepted[n])
        for h in range(inp.H):
            qs = np.concatenate([inp.cq.f64()[n, :a, h], inp.nq.f64()[n, None, h]])
            ks = np.concatenate([inp.ck.f64()[n, :a, h], inp.nk.f64()[n, None, h]])
            vs = np.concatenate([inp.cv.f64()[n, :a, h], inp.nv.f64()[n, None, h]])
            zs = np.concatenate([inp.cz.f64()[n, :a, h], inp.nz.f64()[n, None, h]])
            bs = np.concatenate([inp.cbeta.f64()[n, :a, h], inp.nbeta.f64()[n, None, h]])
            gs = np.stack([gate_h(z) for z in zs])
            ob, Sb = brute.run(qs, ks, vs, gs, bs, inp.state[n, h].astype(np.float64))
            assert _rel(o[n, h], ob[-1]) < 1e-12
            assert _rel(S[n, h], Sb) < 1e-12


@pytest.mark.parametrize("gate", ["bounded", "softplus"])
def test_decode_window_equals_explicit_steps(oracle_mod, gate):
    """Replay, bonus token and the next draft window in one loop (systems page,
    decode): the window drafts' outputs are eq. (1) stepped explicitly past the
    bonus token, and the state kept is the one after the bonus token, whatever
    the window holds."""
    inp = kda_gen.make_decode(12, N=5, H=2, W=4, dtype="bf16", d=128,
                              accepted=[0, 4, 1, 3, 2], W2=3, gate=gate)
    o, ow, S = oracle_mod.decode_window(inp)
    assert ow.shape == (inp.N, 3, inp.H, 128)
    gfun = oracle_mod.gate_softplus if gate == "softplus" else \
        (lambda z, A: oracle_mod.gate(z, A, inp.g_min))
    gate_h = lambda z: gfun(z[None, None, :], inp.A_log[None, h:h + 1])[0, 0]
    cat = lambda c, b, w, n, a, h: np.concatenate([c.f64()[n, :a, h], b.f64()[n, None, h],
                                                    w.f64()[n, :, h]])
    for n in range(inp.N):
        a = int(inp.accepted[n])
        for h in range(inp.H):
            qs = cat(inp.cq, inp.nq, inp.wq, n, a, h)
            ks = cat(inp.ck, inp.nk, inp.wk, n, a, h)
            vs = cat(inp.cv, inp.nv, inp.wv, n, a, h)
            zs = cat(inp.cz, inp.nz, inp.wz, n, a, h)
            bs = cat(inp.cbeta, inp.nbeta, inp.wbeta, n, a, h)
            gs = np.stack([gate_h(z) for z in zs])
            S0 = inp.state[n, h].astype(np.float64)
            ob, _ = brute.run(qs, ks, vs, gs, bs, S0)
            _, Sb = brute.run(qs[:a + 1], ks[:a + 1], vs[:a + 1], gs[:a + 1], bs[:a + 1], S0)
            assert _rel(o[n, h], ob[a]) < 1e-12
            for j in range(3):
                assert _rel(ow[n, j, h], ob[a + 1 + j]) < 1e-12
            assert _rel(S[n, h], Sb) < 1e-12
    # the bonus output and kept state do not depend on the window
    o0, S0_ = oracle_mod.decode(inp)
    assert np.array_equal(o0, o) and np.array_equal(S0_, S)
    # the window's draws come after those of the plain recipe
    plain = kda_gen.make_decode(12, N=5, H=2, W=4, dtype="bf16", d=128, accepted=[0, 4, 1, 3, 2])
    assert np.array_equal(plain.state, inp.state) and np.array_equal(plain.nq.data, inp.nq.data)


# ---------------------------------------------------------------------------
# Raw inputs: q, k normalised and beta = sigmoid(logit) inside the operator
# ("序列维度（下）", section on which form each phase uses: the kernels take q,
# k and beta before L2 normalisation and sigmoid)
# ---------------------------------------------------------------------------
def _raw_case(seed, **kw):
    return kda_gen.make_prefill(seed, 150, 2, "f32", raw=True, lengths=[90, 60], **kw)


def test_raw_inputs_scale_invariance(oracle_mod):
    """Only the direction of q and k counts: scaling each raw q and k row by its
    own positive factor changes nothing."""
    inp = _raw_case(21)
    o, S = oracle_mod.forward(inp)
    rng = _rng(21)
    # powers of two, so that the scaled fp32 rows are exactly proportional
    cq = np.exp2(rng.integers(-8, 9, size=inp.q.shape[:2] + (1,))).astype(np.float32)
    ck = np.exp2(rng.integers(-8, 9, size=inp.k.shape[:2] + (1,))).astype(np.float32)
    scaled = kda_gen.PrefillInputs(
        kda_gen.Tensor(inp.q.data * cq, "f32"), kda_gen.Tensor(inp.k.data * ck, "f32"),
        inp.v, inp.z, inp.beta, inp.A_log, inp.S0, inp.cu_seqlens, inp.g_min, "f32", raw=True)
    o2, S2 = oracle_mod.forward(scaled)
    assert _rel(o2, o) < 1e-12 and _rel(S2, S) < 1e-12


def test_raw_inputs_reduce_to_normalised(oracle_mod):
    """Rows already of unit norm and beta logits of 0 (sigmoid(0) = 1/2 exactly)
    give the operator on those rows with beta = 1/2; zero rows give zero outputs."""
    inp = kda_gen.make_prefill(22, 150, 2, "f32", lengths=[90, 60])   # unit rows (fp32)
    half = np.full(inp.beta.shape, 0.5, dtype=np.float32)
    plain = dataclasses.replace(inp, beta=kda_gen.Tensor(half, "f32"))
    raw = dataclasses.replace(inp, beta=kda_gen.Tensor(np.zeros_like(half), "f32"), raw=True)
    o1, S1 = oracle_mod.forward(plain)
    o2, S2 = oracle_mod.forward(raw)
    assert _rel(o2, o1) < 1e-6 and _rel(S2, S1) < 1e-6   # the fp32 rows are unit to ~1e-7
    zq = dataclasses.replace(raw, q=kda_gen.Tensor(np.zeros_like(inp.q.data), "f32"))
    o3, _ = oracle_mod.forward(zq)
    assert np.all(o3 == 0)


def test_raw_inputs_retrieval(oracle_mod):
    """A large beta logit is beta = 1; with q = k (raw, any norm) the delta rule
    then returns v at every step, as with unit keys and beta = 1."""
    inp = _raw_case(23)
    big = np.full(inp.beta.shape, 60.0, dtype=np.float32)
    r = dataclasses.replace(inp, q=inp.k, beta=kda_gen.Tensor(big, "f32"))
    o, _ = oracle_mod.forward(r)
    assert np.max(np.abs(o - inp.v.f64())) < 1e-10


# ---------------------------------------------------------------------------
# Cost models printed on the SemiAnalysis page ("复杂度分析") and the KCP volume
# ---------------------------------------------------------------------------
def test_cost_models_match_page_numbers():
    import bench
    with open(GOLDEN, encoding="utf-8") as fh:
        gold = json.load(fh)
    f = gold["flashkda_flops_per_chunk"]
    assert bench.flops_model_per_chunk(f["C"], f["D"]) == f["value"]
    b = gold["flashkda_bytes_per_chunk"]
    assert bench.bytes_model_per_chunk(b["C"], b["D"]) == b["value"]
    C, D = b["C"], b["D"]
    assert 3 * 2 * C * D + 2 * (3 * 2 * C * D + 2 * 2 * C * C) + 2 * 2 * C * D == b["value"]
    assert bench.state_bytes(D) == gold["flashkda_state_bytes_per_kernel"]["value"]
    assert bench.decode_flops_per_token(D) == gold["decode_flops_per_head_token"]["value"]
    assert bench.decode_bytes_per_token(D) == gold["decode_bytes_per_head_token"]["value"]
    # KCP pair: (d_k*d_k + d_k*d_v) bf16 elements per head
    pair = 128 * (128 + 128) * 2
    assert pair == gold["kcp_pair_bytes_per_head_bf16"]["value_kb"] * 1024
    assert pair * 96 == gold["kcp_pair_bytes_per_layer"]["value_mb"] * 1024 * 1024
    assert 7 * pair * 96 == gold["kcp_received_per_rank_p8"]["value_mb"] * 1024 * 1024


# ---------------------------------------------------------------------------
# Generators: the recipe (not the method) -- shapes and stated distributions
# ---------------------------------------------------------------------------
def test_generators_recipe():
    inp = kda_gen.workload(0)
    assert inp.q.shape == (256, 2, 128) and inp.dtype == "f32" and inp.S0 is None
    assert np.allclose(np.linalg.norm(inp.q.f32(), axis=-1), 1.0, atol=1e-6)
    assert np.all(inp.A_log == 0)
    small = kda_gen.workload(3, scale_T=20000, scale_H=2)
    lens = np.diff(small.cu_seqlens)
    assert lens.sum() == 20000 and lens.min() >= 64 and small.S0.shape[0] == len(lens)
    assert np.all(small.S0[1:] == 0) and small.S0[0].std() > 0.015
    dec = kda_gen.workload(4, scale_N=16, scale_H=2)
    assert dec.accepted.min() >= 0 and dec.accepted.max() <= 4
    # ties to even; a finite float32 past the largest bf16 (about 3.3895e38) rounds to infinity
    x = np.array([1.0, 1.00390625, 1.005859375, -3.4e38], dtype=np.float32)
    rt = kda_gen.bf16_bits_to_f32(kda_gen.f32_to_bf16_bits(x))
    assert rt[0] == 1.0 and rt[1] == 1.0 and rt[2] == 1.0078125
    assert rt[3] == -np.inf
