"""GPU parity at the largest head count the ABI accepts (H = 65535).

The kernels address one 64-token chunk of one head with 32-bit offsets, which is
what bounds H: at H = 65535 the per-chunk input spans reach 1.06e9 bytes for bf16
and 2.11e9 bytes for fp32 inputs, just under 2^31.  These tests run every prefill
path and the decode step there, on a document of 65 tokens (one full chunk and
a one-token tail), and compare sampled heads (every residue mod 8, both ends)
with the oracle.

The inputs are seeded and synthetic: 1021 heads drawn with the usual recipe and
repeated along the head axis (a period that is not a power of two, so an offset
that wrapped at one would read other data), with a gate parameter A_h drawn
for every head, so no two heads with the same data have the same decay.
"""
import dataclasses

import numpy as np
import pytest

import kda_gen
import oracle
from kda_testlib import TOL_BF16, TOL_BF16_STORAGE, TOL_F32, oracle_forward, rel_l2_slices

pytestmark = pytest.mark.gpu

H_MAX = 65535
PERIOD = 1021
HEADS = [0, 1, 2, 3, 4, 5, 6, 7, 1020, 1021, 32767, 32768, 65527, 65534]


def _tile(t, axis, H):
    idx = np.arange(H) % PERIOD
    return kda_gen.Tensor(np.take(t.data, idx, axis=axis), t.dtype)


def _prefill_inputs(dtype, T=65):
    base = kda_gen.make_prefill(71, T, PERIOD, dtype)
    A = np.random.default_rng(72).standard_normal(H_MAX).astype(np.float32) * np.float32(0.5)
    return dataclasses.replace(base, q=_tile(base.q, 1, H_MAX), k=_tile(base.k, 1, H_MAX),
                               v=_tile(base.v, 1, H_MAX), z=_tile(base.z, 1, H_MAX),
                               beta=_tile(base.beta, 1, H_MAX), A_log=A)


def _compare(tag, o, S, inp, o_tol, s_tol):
    o_ref, S_ref = oracle_forward(inp, heads=HEADS)
    eo, _ = rel_l2_slices(o, o_ref, inp.cu_seqlens)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"    {tag}: O {eo:.3e} S {es:.3e} over heads {HEADS}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= o_tol and es <= s_tol, (tag, eo, es)


def _run_prefill(inp, path):
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import gpu_inputs
    t = gpu_inputs(inp)
    args = (t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min, None, None, None)
    if path == "segment_scan":
        # two segments: the workspace is sized for either arithmetic path, and the
        # fp32 one would cut 65 tokens into 65 segments of pairs at this H
        o, S = kda.kda_segment_scan(*args, n_segments=2)
    else:
        o, S = kda.kda_chunk_fwd(*args, compute=1 if path == "fp32" else 0,
                                 workspace=False if path == "fused" else None)
    torch.cuda.synchronize()
    hs = torch.tensor(HEADS, device=o.device)
    o_s = kda_gen.from_torch(o.index_select(1, hs))
    S_s = kda_gen.from_torch(S.index_select(1, hs))
    del t, o, S
    torch.cuda.empty_cache()
    return o_s, S_s


def test_max_heads_prefill_bf16():
    print(f"[case] prefill T=65 H={H_MAX} bf16: two kernels, fused, fp32 arithmetic, "
          "segment scan", flush=True)
    inp = _prefill_inputs("bf16")
    for path in ("two_kernel", "fused", "fp32", "segment_scan"):
        print(f"    path {path}", flush=True)
        o, S = _run_prefill(inp, path)
        tols = (TOL_F32 + TOL_BF16_STORAGE, TOL_F32) if path == "fp32" else (TOL_BF16, TOL_BF16)
        _compare(path, o, S, inp, *tols)


def test_max_heads_prefill_fp32_inputs():
    """fp32 inputs: the widest per-chunk spans (2.11e9 bytes) of any path."""
    print(f"[case] prefill T=65 H={H_MAX} fp32 inputs", flush=True)
    inp = _prefill_inputs("f32")
    o, S = _run_prefill(inp, "fp32")
    _compare("fp32 inputs", o, S, inp, TOL_F32, TOL_F32)


def _slice_decode(inp, hs):
    """The decode inputs of heads hs only (for the oracle)."""
    def sl(t, axis):
        return kda_gen.Tensor(np.take(t.data, hs, axis=axis), t.dtype)
    return dataclasses.replace(inp, state=inp.state[:, hs], cq=sl(inp.cq, 2), ck=sl(inp.ck, 2),
                               cv=sl(inp.cv, 2), cz=sl(inp.cz, 2), cbeta=sl(inp.cbeta, 2),
                               nq=sl(inp.nq, 1), nk=sl(inp.nk, 1), nv=sl(inp.nv, 1),
                               nz=sl(inp.nz, 1), nbeta=sl(inp.nbeta, 1), A_log=inp.A_log[hs])


def test_max_heads_decode():
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import decode_gpu_inputs
    print(f"[case] decode N=3 H={H_MAX} W=4", flush=True)
    base = kda_gen.make_decode(73, 3, PERIOD, 4, "bf16", accepted=[0, 2, 4])
    A = np.random.default_rng(74).standard_normal(H_MAX).astype(np.float32) * np.float32(0.5)
    idx = np.arange(H_MAX) % PERIOD
    inp = dataclasses.replace(base, state=np.ascontiguousarray(base.state[:, idx]),
                              cq=_tile(base.cq, 2, H_MAX), ck=_tile(base.ck, 2, H_MAX),
                              cv=_tile(base.cv, 2, H_MAX), cz=_tile(base.cz, 2, H_MAX),
                              cbeta=_tile(base.cbeta, 2, H_MAX), nq=_tile(base.nq, 1, H_MAX),
                              nk=_tile(base.nk, 1, H_MAX), nv=_tile(base.nv, 1, H_MAX),
                              nz=_tile(base.nz, 1, H_MAX), nbeta=_tile(base.nbeta, 1, H_MAX),
                              A_log=A)
    t = decode_gpu_inputs(inp)
    o = kda.kda_decode_step(t["state"], t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"],
                            t["accepted"], t["nq"], t["nk"], t["nv"], t["nz"], t["nbeta"],
                            t["A_log"], inp.g_min)
    torch.cuda.synchronize()
    hs = torch.tensor(HEADS, device=o.device)
    o_s = kda_gen.from_torch(o.index_select(1, hs))
    S_s = kda_gen.from_torch(t["state"].index_select(1, hs))
    del t, o
    torch.cuda.empty_cache()
    o_ref, S_ref = oracle.decode(_slice_decode(inp, HEADS))
    eo, _ = rel_l2_slices(o_s[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S_s, S_ref, axis_tokens=False)
    print(f"    o {eo:.3e} state {es:.3e} over heads {HEADS}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_F32
