"""GPU parity on the five named workloads at their full sizes.

Each runs the HIP path through the C ABI in the launch configuration bench.py
uses and compares with the CPU oracle on the same seeded inputs, over every
head and every document: the maximum relative L2 error per (document, head)
slice (the stated tolerance) and, for outputs, the worst single token against
its slice's RMS token norm (kda_testlib.token_err_max).
"""
import numpy as np
import pytest

import kda_gen
import oracle
from kda_testlib import (TOK_BF16, TOK_F32, TOL_BF16, TOL_BF16_STORAGE, TOL_F32, gpu_chunk_fwd,
                         gpu_decode, gpu_decode_window, gpu_inputs, gpu_segment_scan,
                         oracle_forward, rel_l2_slices, token_err_max)

pytestmark = pytest.mark.gpu


def _report(tag, o, o_ref, S, S_ref, cu, tok_bound=TOK_BF16):
    """Print and return the slice maxima; assert the per-token bound on O."""
    eo, go = rel_l2_slices(o, o_ref, cu)
    es, gs = rel_l2_slices(S, S_ref, axis_tokens=False)
    et = token_err_max(o, o_ref, cu)
    print(f"[{tag}] O max {eo:.3e} (global {go:.3e}, worst token {et:.3e}) | "
          f"S max {es:.3e} (global {gs:.3e})", flush=True)
    assert et <= tok_bound, (tag, et)
    return eo, es


def test_tiny_fp32_workload():
    inp = kda_gen.workload(0)
    print("[case] tiny fp32 T=256 H=2", flush=True)
    o, S = gpu_chunk_fwd(inp)
    o_ref, S_ref = oracle.forward(inp)
    eo, es = _report("tiny", o, o_ref, S, S_ref, inp.cu_seqlens, tok_bound=TOK_F32)
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
    eo, es = _report("fp32 arithmetic", o32, o_ref, S32, S_ref, inp.cu_seqlens,
                     tok_bound=TOK_F32 + TOL_BF16_STORAGE)
    assert eo <= TOL_F32 + TOL_BF16_STORAGE and es <= TOL_F32


def test_long_prefill_segment_scan_workload():
    """One TP rank's 8 heads over 262144 tokens: the default plan (one (segment,
    head) per compute unit, one-level scan) and one segment per compute unit
    (256, two-level scan); the result must match a single serial pass (the
    oracle, and the chunk kernel)."""
    import linear_attention_fwd_amd as kda
    inp = kda_gen.workload(2)
    n_cu = kda.kda_default_segments()
    t = gpu_inputs(inp)
    o_ref, S_ref = oracle_forward(inp, group=8)
    for n_seg in (0, n_cu):
        print(f"[case] long prefill T=262144 H=8, n_segments={n_seg}", flush=True)
        o, S = gpu_segment_scan(inp, n_segments=n_seg, t=t)
        eo, es = _report("segment scan vs oracle", o, o_ref, S, S_ref, inp.cu_seqlens)
        assert eo <= TOL_BF16 and es <= TOL_BF16
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    eo1, es1 = _report("serial chunk kernel vs oracle", o1, o_ref, S1, S_ref, inp.cu_seqlens)
    assert eo1 <= TOL_BF16 and es1 <= TOL_BF16


def test_long_prefill_long_memory_segment_scan():
    """The long-prefill shape (T=262144, H=8; the default plan of 32 segments
    and one segment per compute unit) with decays of about 1e-4 to 5e-3 per
    token (z ~ N(-9, 1), A = 0): states remember across segments and groups, so
    the pairs and the scans decide the outputs (both plans), unlike under
    the workload's own decays (about -2.5 per token), which forget an entry
    state within a few tokens."""
    inp = kda_gen.make_prefill(52, 262144, 8, "bf16", A_std=0.0, z_mean=-9.0, z_std=1.0,
                               s0_std=0.05, s0_docs="all")
    g = oracle.gate(inp.z.f64()[:4096:64], inp.A_log, inp.g_min)
    print(f"[case] long prefill, long memory: per-token decay median {np.median(-g):.1e}, "
          f"90% in [{np.quantile(-g, 0.05):.1e}, {np.quantile(-g, 0.95):.1e}]", flush=True)
    import linear_attention_fwd_amd as kda
    t = gpu_inputs(inp)
    o_ref, S_ref = oracle_forward(inp, group=8)
    for n_seg in (0, kda.kda_default_segments()):
        print(f"    n_segments={n_seg}", flush=True)
        o, S = gpu_segment_scan(inp, n_segments=n_seg, t=t)
        eo, es = _report("segment scan vs oracle", o, o_ref, S, S_ref, inp.cu_seqlens)
        assert eo <= TOL_BF16 and es <= TOL_BF16
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    eo1, es1 = _report("serial chunk kernel vs oracle", o1, o_ref, S1, S_ref, inp.cu_seqlens)
    assert eo1 <= TOL_BF16 and es1 <= TOL_BF16


def test_packed_varlen_workload():
    inp = kda_gen.workload(3)
    print(f"[case] packed varlen T=65536 H=96, {inp.N} documents", flush=True)
    o, S = gpu_chunk_fwd(inp)
    o_ref, S_ref = oracle_forward(inp, group=16)
    eo, es = _report("varlen, all 96 heads", o, o_ref, S, S_ref, inp.cu_seqlens)
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


# ---------------------------------------------------------------------------
# the next items at the sizes bench.py times them
# ---------------------------------------------------------------------------
def test_single_sequence_checkpoints_workload():
    """Checkpoints every 512 tokens of the single-sequence workload (15 of them)
    against the oracle on all heads: the oracle runs the sequence piece by
    piece, each piece from the state the previous one ends with, and the state
    after each piece is the checkpoint.  O and the final state are those of
    kda_chunk_fwd, bit for bit."""
    import linear_attention_fwd_amd as kda
    import torch
    inp = kda_gen.workload(1)
    interval = 512
    print(f"[case] checkpoints every {interval} tokens, T=8192 H=96", flush=True)
    t = gpu_inputs(inp)
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    o2, S2, ck = kda.kda_chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["z"], t["beta"],
                                               interval, t["A_log"], inp.g_min)
    torch.cuda.synchronize()
    assert np.array_equal(o1, kda_gen.from_torch(o2)) and np.array_equal(S1, kda_gen.from_torch(S2))
    ck = kda_gen.from_torch(ck)
    assert ck.shape[0] == kda.kda_checkpoint_count(1, inp.T, interval)
    assert all(kda.checkpoint_index(None, 0, j, interval) == j - 1 < ck.shape[0] for j in range(1, 16))
    worst = 0.0
    for h0 in range(0, inp.H, 16):
        heads = list(range(h0, h0 + 16))
        q, k, v, b = (x.f64()[:, heads] for x in (inp.q, inp.k, inp.v, inp.beta))
        g = oracle.gate(inp.z.f64()[:, heads], inp.A_log[heads], inp.g_min)
        S = None
        for j in range(1, inp.T // interval):
            a, e = (j - 1) * interval, j * interval
            _, S = oracle.recurrent(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], S)
            err, _ = rel_l2_slices(ck[j - 1][None, heads], S, axis_tokens=False)
            worst = max(worst, err)
    print(f"    15 checkpoints x {inp.H} heads, max rel L2 {worst:.3e}", flush=True)
    assert worst <= TOL_BF16


def test_unbounded_gate_single_sequence_workload():
    """The single-sequence workload with the unbounded softplus gate in place of the
    bounded one (same logits), against the oracle on all heads."""
    import dataclasses
    import linear_attention_fwd_amd as kda
    import torch
    inp = dataclasses.replace(kda_gen.workload(1), gate="softplus")
    print("[case] unbounded gate, T=8192 H=96", flush=True)
    t = gpu_inputs(inp)
    o, S = kda.kda_chunk_fwd_unbounded(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"])
    torch.cuda.synchronize()
    o, S = kda_gen.from_torch(o), kda_gen.from_torch(S)
    o_ref, S_ref = oracle_forward(inp, group=16)
    eo, es = _report("unbounded gate, all 96 heads", o, o_ref, S, S_ref, inp.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_window_workload():
    """The decode workload with a next window of 4 drafts (the configuration
    bench.py times): bonus output and state bit for bit those of kda_decode_step,
    the window's outputs against the oracle."""
    inp = kda_gen.make_decode(4, 512, 96, 4, "bf16", W2=4)
    print("[case] decode N=512 H=96 W=4 + next window of 4", flush=True)
    o_ref, ow_ref, S_ref = oracle.decode_window(inp)
    o, ow, S = gpu_decode_window(inp)
    o1, S1 = gpu_decode(inp)
    assert np.array_equal(o, o1) and np.array_equal(S, S1)
    ew = max(rel_l2_slices(ow[:, j][:, :, None], ow_ref[:, j][:, :, None], axis_tokens=False)[0]
             for j in range(4))
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"[decode window] window o max {ew:.3e} | state max {es:.3e}", flush=True)
    assert ew <= TOL_BF16 and es <= TOL_F32


def test_raw_inputs_workloads():
    """The single-sequence and decode workloads drawn raw (q, k unnormalised, beta
    logits, from the same draws), normalised inside the kernels, against the
    oracle that normalises them (all heads)."""
    import linear_attention_fwd_amd as kda
    import torch
    pre = kda_gen.make_prefill(1, 8192, 96, "bf16", A_std=0.5, raw=True)
    print("[case] raw inputs, T=8192 H=96 and decode N=512 H=96", flush=True)
    t = gpu_inputs(pre)
    o, S = gpu_chunk_fwd(pre, t=t)
    o_ref, S_ref = oracle_forward(pre, group=16)
    eo, es = _report("raw prefill, all 96 heads", o, o_ref, S, S_ref, pre.cu_seqlens)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    dec = kda_gen.make_decode(4, 512, 96, 4, "bf16", raw=True)
    od_ref, Sd_ref = oracle.decode(dec)
    od, Sd = gpu_decode(dec)
    e1, _ = rel_l2_slices(od[:, :, None], od_ref[:, :, None], axis_tokens=False)
    e2, _ = rel_l2_slices(Sd, Sd_ref, axis_tokens=False)
    print(f"[raw decode] o max {e1:.3e} | state max {e2:.3e}", flush=True)
    assert e1 <= TOL_BF16 and e2 <= TOL_F32
