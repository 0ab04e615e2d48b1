"""GPU parity on the five named workloads at their full sizes.

Each runs the HIP path through the C ABI in the launch configuration bench.py
uses and compares with the CPU oracle on the same seeded inputs.  Where the
oracle would take long, outputs are compared on a sample of heads (every
document of those heads), the rest is checked for finiteness.
"""
import numpy as np
import pytest

import kda_gen
import oracle
from kda_testlib import (TOL_BF16, TOL_BF16_STORAGE, TOL_F32, gpu_chunk_fwd, gpu_decode,
                         gpu_inputs, gpu_segment_scan, oracle_forward, rel_l2_slices)

pytestmark = pytest.mark.gpu


def _report(tag, o, o_ref, S, S_ref, cu):
    eo, go = rel_l2_slices(o, o_ref, cu)
    es, gs = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"[{tag}] O max {eo:.3e} (global {go:.3e}) | S max {es:.3e} (global {gs:.3e})",
          flush=True)
    return eo, es


def test_tiny_fp32_workload():
    inp = kda_gen.workload(0)
    print("[case] tiny fp32 T=256 H=2", flush=True)
    o, S = gpu_chunk_fwd(inp)
    o_ref, S_ref = oracle.forward(inp)
    eo, es = _report("tiny", o, o_ref, S, S_ref, inp.cu_seqlens)
    assert eo <= TOL_F32 and es <= TOL_F32


def test_single_sequence_workload():
    inp = kda_gen.workload(1)
    print("[case] single sequence T=8192 H=96 bf16", flush=True)
    t = gpu_inputs(inp)
    o_ref, S_ref = oracle_forward(inp, group=16)
    o, S = gpu_chunk_fwd(inp, t=t)
    eo, es = _report("bf16, prep + recurrence kernels", o, o_ref, S, S_ref, inp.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    of, Sf = gpu_chunk_fwd(inp, t=t, fused=True)
    eo, es = _report("bf16, fused kernel", of, o_ref, Sf, S_ref, inp.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    o32, S32 = gpu_chunk_fwd(inp, compute=1, t=t)
    eo, es = _report("fp32 arithmetic", o32, o_ref, S32, S_ref, inp.cu_seqlens)
    assert eo <= TOL_F32 + TOL_BF16_STORAGE and es <= TOL_F32


def test_long_prefill_segment_scan_workload():
    """One TP rank's 8 heads over 262144 tokens, one segment per compute unit; the
    result must match a single serial pass (the oracle, and the chunk kernel)."""
    import linear_attention_fwd_amd as kda
    inp = kda_gen.workload(2)
    n_seg = kda.kda_default_segments()
    print(f"[case] long prefill T=262144 H=8, {n_seg} segments", flush=True)
    t = gpu_inputs(inp)
    o, S = gpu_segment_scan(inp, n_segments=0, t=t)
    o_ref, S_ref = oracle_forward(inp, group=8)
    eo, es = _report("segment scan vs oracle", o, o_ref, S, S_ref, inp.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    eo1, es1 = _report("serial chunk kernel vs oracle", o1, o_ref, S1, S_ref, inp.cu_seqlens)
    assert eo1 <= TOL_BF16 and es1 <= TOL_BF16


def test_packed_varlen_workload():
    inp = kda_gen.workload(3)
    print(f"[case] packed varlen T=65536 H=96, {inp.N} documents", flush=True)
    o, S = gpu_chunk_fwd(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    heads = list(range(0, 96, 6))  # 16 sampled heads, every document
    o_ref, S_ref = oracle_forward(inp, heads=heads, group=16)
    eo, es = _report("varlen, 16 sampled heads", o[:, heads], o_ref, S[:, heads], S_ref,
                     inp.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_workload():
    inp = kda_gen.workload(4)
    print(f"[case] decode N=512 H=96 W=4", flush=True)
    o_ref, S_ref = oracle.decode(inp)
    o, S = gpu_decode(inp)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"[decode] o max {eo:.3e} | state max {es:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_F32
