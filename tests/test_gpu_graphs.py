"""The entry points under HIP graph capture.

The library enqueues kernels only (no allocation, memset, copy or
synchronisation), so with the outputs and workspaces allocated beforehand a
whole prefill or decode step can be captured once and replayed.  Each test
captures the calls, then replays the graph several times with new inputs
written into the captured tensors by ordinary (eager) work in between, and
checks every replay bit for bit against the same calls made eagerly.
"""
import numpy as np
import pytest

import kda_gen
from kda_testlib import TOL_BF16, gpu_inputs, oracle_forward, rel_l2_slices

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _prefill_draw(seed):
    return kda_gen.make_prefill(seed, 700, 4, "bf16", lengths=[130, 0, 257, 1, 0, 312],
                                s0_std=0.02, s0_docs="all")


def test_prefill_graph_replays():
    """kda_chunk_fwd_noalloc, kda_chunk_fwd with a caller workspace and
    kda_segment_scan in one captured graph; every replay equals the eager calls on
    the same inputs, and the first also matches the oracle."""
    import torch
    import linear_attention_fwd_amd as kda
    inp = _prefill_draw(81)
    print(f"[case] graph prefill T={inp.T} H={inp.H} N={inp.N}", flush=True)
    t = gpu_inputs(inp)
    args = lambda: (t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min, t["S0"],
                    t["cu"], t["cu_host"])
    ws = torch.empty(kda.kda_chunk_fwd_workspace_size(inp.N, inp.T, inp.H), dtype=torch.uint8,
                     device="cuda")
    n_seg = 5
    ws_scan = torch.empty(kda.kda_segment_scan_workspace_size(inp.N, inp.T, inp.H, n_seg),
                          dtype=torch.uint8, device="cuda")
    o = [torch.empty((inp.T, inp.H, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    S = [torch.empty((inp.N, inp.H, 128, 128), dtype=torch.float32, device="cuda")
         for _ in range(3)]

    def calls():
        kda.kda_chunk_fwd_noalloc(*args(), o=o[0], final_state=S[0])
        kda.kda_chunk_fwd(*args(), o=o[1], final_state=S[1], workspace=ws)
        kda.kda_segment_scan(*args(), n_segments=n_seg, o=o[2], final_state=S[2],
                             workspace=ws_scan)

    calls()  # first calls outside capture (the no-allocation scratch is looked up here)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        new = _prefill_draw(82 + r)
        for name in ("q", "k", "v", "z", "beta"):
            t[name].copy_(kda_gen.to_torch(getattr(new, name), "cuda"))
        t["S0"].copy_(torch.from_numpy(new.S0).to("cuda"))
        t["A_log"].copy_(torch.from_numpy(new.A_log).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [(kda_gen.from_torch(o[i]), kda_gen.from_torch(S[i])) for i in range(3)]
        o_e, S_e = kda.kda_chunk_fwd(*args(), workspace=ws)
        o_s, S_s = kda.kda_segment_scan(*args(), n_segments=n_seg, workspace=ws_scan)
        torch.cuda.synchronize()
        o_e, S_e = kda_gen.from_torch(o_e), kda_gen.from_torch(S_e)
        o_s, S_s = kda_gen.from_torch(o_s), kda_gen.from_torch(S_s)
        print(f"    replay {r}", flush=True)
        for i, (oo, SS) in enumerate(got[:2]):
            assert np.array_equal(oo, o_e) and np.array_equal(SS, S_e), (r, i)
        assert np.array_equal(got[2][0], o_s) and np.array_equal(got[2][1], S_s), r
        if r == 0:
            o_ref, S_ref = oracle_forward(new)
            eo, _ = rel_l2_slices(o_e, o_ref, new.cu_seqlens)
            es, _ = rel_l2_slices(S_e, S_ref, axis_tokens=False)
            print(f"    O {eo:.3e}  S {es:.3e}", flush=True)
            assert eo <= TOL_BF16 and es <= TOL_BF16


def test_segment_scan_default_plan_graph_replays():
    """kda_segment_scan with the default plan (n_segments = 0; at H = 8 one
    (segment, head) per compute unit, scanned in one level), captured once: every
    replay on new inputs equals the same eager call bit for bit."""
    import torch
    import linear_attention_fwd_amd as kda

    def draw(seed):
        return kda_gen.make_prefill(seed, 1500, 8, "bf16", lengths=[130, 0, 700, 1, 0, 669],
                                    s0_std=0.02, s0_docs="all")

    inp = draw(91)
    print(f"[case] graph segment scan, default plan, T={inp.T} H={inp.H} N={inp.N}", flush=True)
    t = gpu_inputs(inp)
    args = lambda: (t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min, t["S0"],
                    t["cu"], t["cu_host"])
    ws = torch.empty(kda.kda_segment_scan_workspace_size(inp.N, inp.T, inp.H, 0),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((inp.T, inp.H, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((inp.N, inp.H, 128, 128), dtype=torch.float32, device="cuda")
    kda.kda_segment_scan(*args(), n_segments=0, o=o, final_state=S, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.kda_segment_scan(*args(), n_segments=0, o=o, final_state=S, workspace=ws)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        new = draw(92 + r)
        for name in ("q", "k", "v", "z", "beta"):
            t[name].copy_(kda_gen.to_torch(getattr(new, name), "cuda"))
        t["S0"].copy_(torch.from_numpy(new.S0).to("cuda"))
        t["A_log"].copy_(torch.from_numpy(new.A_log).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_S = kda_gen.from_torch(o), kda_gen.from_torch(S)
        o_e, S_e = kda.kda_segment_scan(*args(), n_segments=0, workspace=ws)
        torch.cuda.synchronize()
        o_e, S_e = kda_gen.from_torch(o_e), kda_gen.from_torch(S_e)
        print(f"    replay {r}", flush=True)
        assert np.array_equal(got_o, o_e) and np.array_equal(got_S, S_e), r
        if r == 0:
            o_ref, S_ref = oracle_forward(new)
            eo, _ = rel_l2_slices(o_e, o_ref, new.cu_seqlens)
            es, _ = rel_l2_slices(S_e, S_ref, axis_tokens=False)
            print(f"    O {eo:.3e}  S {es:.3e}", flush=True)
            assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_graph_replays():
    """The decode step with the next window, captured once: each replay advances
    the states in place exactly as the same eager call does on a copy of them."""
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import decode_gpu_inputs
    inp = kda_gen.make_decode(83, 24, 4, 4, "bf16", W2=3)
    print(f"[case] graph decode N={inp.N} H={inp.H} W={inp.W} W2={inp.W2}", flush=True)
    t = decode_gpu_inputs(inp)
    names = ("cq", "ck", "cv", "cz", "cbeta", "nq", "nk", "nv", "nz", "nbeta",
             "wq", "wk", "wv", "wz", "wbeta")
    o = torch.empty((inp.N, inp.H, 128), dtype=torch.bfloat16, device="cuda")
    ow = torch.empty((inp.N, inp.W2, inp.H, 128), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(state, out, out_w):
        kda.kda_decode_step_window(state, t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"],
                                   t["accepted"], t["nq"], t["nk"], t["nv"], t["nz"], t["nbeta"],
                                   t["wq"], t["wk"], t["wv"], t["wz"], t["wbeta"], t["A_log"],
                                   inp.g_min, o=out, o_window=out_w, err_flag=err)

    shadow = t["state"].clone()  # advanced eagerly beside the graph
    step(shadow, torch.empty_like(o), torch.empty_like(ow))  # outside capture
    t["state"].copy_(shadow)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(t["state"], o, ow)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        new = kda_gen.make_decode(84 + r, 24, 4, 4, "bf16", W2=3)
        for name in names:
            t[name].copy_(kda_gen.to_torch(getattr(new, name), "cuda"))
        t["accepted"].copy_(torch.from_numpy(new.accepted).to("cuda"))
        t["A_log"].copy_(torch.from_numpy(new.A_log).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        o_e, ow_e = torch.empty_like(o), torch.empty_like(ow)
        step(shadow, o_e, ow_e)
        torch.cuda.synchronize()
        print(f"    replay {r}", flush=True)
        assert torch.equal(t["state"], shadow), r
        assert torch.equal(o, o_e) and torch.equal(ow, ow_e), r
    assert int(err.item()) == 0
