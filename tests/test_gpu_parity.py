"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes here run in seconds on the oracle and still span several chunks, ragged
tails, empty documents and the gate's extreme regimes.  The full workloads are
in test_gpu_workloads.py.  Tolerance: max relative L2 error per (document,
head) slice of O and of the final state, 1e-2 for bf16-MFMA arithmetic and
1e-4 for the fp32 verification arithmetic.
"""
import numpy as np
import pytest

import kda_gen
from kda_testlib import (TOL_BF16, TOL_BF16_STORAGE, TOL_F32, gpu_chunk_fwd, gpu_decode,
                         gpu_decode_window, gpu_segment_scan, gpu_chunk_fwd_unbounded,
                         decode_gpu_inputs, oracle_forward, rel_l2_slices)
import oracle

pytestmark = pytest.mark.gpu


def _case(inp, compute):
    print(f"[case] T={inp.T} H={inp.H} N={inp.N} dtype={inp.dtype} compute={compute}", flush=True)


def _tols(inp, compute):
    """(tolerance on O, tolerance on the final state)."""
    if inp.dtype == "f32" or compute == 1:
        o_tol = TOL_F32 if inp.dtype == "f32" else TOL_F32 + TOL_BF16_STORAGE
        return o_tol, TOL_F32
    return TOL_BF16, TOL_BF16


def _check_prefill(inp, o, S, tols, ref=None):
    o_ref, S_ref = ref if ref is not None else oracle_forward(inp)
    eo, go = rel_l2_slices(o, o_ref, inp.cu_seqlens)
    es, gs = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"    O: max {eo:.3e} global {go:.3e} | S: max {es:.3e} global {gs:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= tols[0], eo
    assert es <= tols[1], es
    return eo, es


PREFILL_CASES = {
    # name: (generator kwargs)
    "tiny_fp32_workload": dict(seed=0, T=256, H=2, dtype="f32", A_std=0.0),
    "ragged_tail_bf16": dict(seed=21, T=300, H=4, dtype="bf16", s0_std=0.02, s0_docs="all"),
    "single_token": dict(seed=22, T=1, H=3, dtype="bf16", s0_std=0.02, s0_docs="all"),
    "slow_decay_long_memory": dict(seed=23, T=700, H=2, dtype="bf16", z_mean=-6.0,
                                   s0_std=0.05, s0_docs="all"),
    "decay_near_bound": dict(seed=24, T=256, H=2, dtype="bf16", z_mean=8.0),
    "varlen_with_empty_docs": dict(seed=25, T=400, H=3, dtype="bf16",
                                   lengths=[5, 0, 130, 64, 1, 200, 0], s0_std=0.02,
                                   s0_docs="all"),
    "varlen_fp32": dict(seed=26, T=333, H=2, dtype="f32", lengths=[100, 0, 64, 169],
                        s0_std=0.1, s0_docs="all"),
}


@pytest.mark.parametrize("name", sorted(PREFILL_CASES))
def test_chunk_fwd_matches_oracle(name):
    kw = dict(PREFILL_CASES[name])
    seed, T, H = kw.pop("seed"), kw.pop("T"), kw.pop("H")
    inp = kda_gen.make_prefill(seed, T, H, **kw)
    ref = oracle_forward(inp)
    # bf16 inputs: the two-kernel path (workspace), the fused kernel, fp32 arithmetic
    runs = ((0, False),) if inp.dtype == "f32" else ((0, False), (0, True), (1, False))
    for compute, fused in runs:
        _case(inp, compute)
        print(f"    path={'fused' if fused or inp.dtype == 'f32' or compute else 'prep+recurrence'}",
              flush=True)
        o, S = gpu_chunk_fwd(inp, compute=compute, fused=fused)
        _check_prefill(inp, o, S, _tols(inp, compute), ref)


def test_two_kernel_path_matches_fused_kernel():
    """Both prefill paths run the same stage code; they agree to well below the
    bf16 tolerance (with identical compiled arithmetic, bit for bit)."""
    inp = kda_gen.make_prefill(33, 777, 3, "bf16", lengths=[64, 1, 0, 300, 412],
                               s0_std=0.02, s0_docs="all")
    o1, S1 = gpu_chunk_fwd(inp)
    o2, S2 = gpu_chunk_fwd(inp, fused=True)
    print(f"    identical O: {np.array_equal(o1, o2)}, identical S: {np.array_equal(S1, S2)}",
          flush=True)
    eo, _ = rel_l2_slices(o1, o2, inp.cu_seqlens)
    es, _ = rel_l2_slices(S1, S2, axis_tokens=False)
    assert eo <= 1e-3 and es <= 1e-3, (eo, es)


def test_prep_then_recurrence_equals_chunk_fwd():
    """The two halves called on their own give kda_chunk_fwd's result exactly."""
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import gpu_inputs
    inp = kda_gen.make_prefill(34, 450, 3, "bf16", lengths=[200, 0, 250], s0_std=0.02,
                               s0_docs="all")
    t = gpu_inputs(inp)
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    ws = torch.empty(kda.kda_chunk_fwd_workspace_size(inp.N, inp.T, inp.H), dtype=torch.uint8,
                     device="cuda")
    kda.kda_chunk_prep(t["q"], t["k"], t["z"], t["beta"], ws, t["A_log"], inp.g_min, t["cu"],
                       t["cu_host"])
    o2, S2 = kda.kda_chunk_recurrence(t["v"], ws, t["S0"], t["cu"], t["cu_host"])
    torch.cuda.synchronize()
    assert np.array_equal(o1, kda_gen.from_torch(o2))
    assert np.array_equal(S1, kda_gen.from_torch(S2))


def _expected_doc_order(lengths):
    """Longest first by chunk count rounded down to its leading 4 bits, empty
    documents last, input order among equal keys."""
    def key(n):
        c = (n + 63) // 64
        if c == 0:
            return 255
        e = c.bit_length() - 1
        m = (c >> (e - 3)) & 7 if e >= 3 else (c << (3 - e)) & 7
        return 254 - min(8 * e + m, 254)
    return sorted(range(len(lengths)), key=lambda d: (key(lengths[d]), d))


@pytest.mark.parametrize("case", ["unsorted_with_empty", "many_documents", "mostly_empty", "sorted"])
def test_document_order(case):
    """kda_chunk_prep writes the order in which the recurrence takes the
    documents after the chunk images: longest first, a permutation of [0, N);
    documents already in that order leave it unwritten."""
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import gpu_inputs
    rng = np.random.default_rng(36)
    lengths = {"unsorted_with_empty": [5, 0, 130, 64, 1, 200, 0, 4000, 65],
               "many_documents": [int(x) for x in rng.integers(0, 300, size=700)] + [0, 9000],
               "mostly_empty": [0] * 300 + [500] + [0] * 213,
               "sorted": [900, 640, 577, 64, 10, 0]}[case]
    inp = kda_gen.make_prefill(36, int(sum(lengths)), 1, "bf16", lengths=lengths)
    _case(inp, 0)
    t = gpu_inputs(inp)
    nbytes = kda.kda_chunk_fwd_workspace_size(inp.N, inp.T, inp.H)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    kda.kda_chunk_prep(t["q"], t["k"], t["z"], t["beta"], ws, t["A_log"], inp.g_min, t["cu"],
                       t["cu_host"])
    torch.cuda.synchronize()
    off = (inp.T // 64 + inp.N) * inp.H * 62464
    assert nbytes == off + (4 * inp.N + 255) // 256 * 256
    order = ws[off:off + 4 * inp.N].cpu().numpy().view(np.int32)
    if case == "sorted":
        assert np.all(order == -1)
        return
    assert np.array_equal(np.sort(order), np.arange(inp.N))
    assert order.tolist() == _expected_doc_order(lengths)


def test_document_order_changes_no_result():
    """Hundreds of documents around two long ones (the order kernel places
    them over two passes) through the whole prefill, against the oracle; and
    the same documents packed in another order (already longest first, so no
    order is written) give bit-identical results per document.  Lengths start
    at 40 tokens: the max over (document, head) slices of a few tokens each
    samples the far tail of bf16 operand rounding on outputs that cancel."""
    rng = np.random.default_rng(37)
    lengths = [int(x) for x in rng.integers(40, 120, size=300)]
    lengths[17], lengths[250] = 2000, 700
    lengths[5] = lengths[100] = 0
    inp = kda_gen.make_prefill(37, int(sum(lengths)), 2, "bf16", lengths=lengths, s0_std=0.02,
                               s0_docs="all")
    _case(inp, 0)
    o, S = gpu_chunk_fwd(inp)
    _check_prefill(inp, o, S, _tols(inp, 0))
    cu = inp.cu_seqlens
    perm = sorted(range(inp.N), key=lambda d: -((lengths[d] + 63) // 64))
    cu2 = np.concatenate([[0], np.cumsum([lengths[d] for d in perm])]).astype(np.int32)

    def packed(x):
        return np.concatenate([x[cu[d]:cu[d + 1]] for d in perm])
    inp2 = kda_gen.PrefillInputs(*(kda_gen.Tensor(packed(x.data), x.dtype) for x in
                                   (inp.q, inp.k, inp.v, inp.z, inp.beta)), inp.A_log,
                                 inp.S0[perm], cu2, inp.g_min, inp.dtype)
    o2, S2 = gpu_chunk_fwd(inp2)
    for i, d in enumerate(perm):
        assert np.array_equal(o2[cu2[i]:cu2[i + 1]], o[cu[d]:cu[d + 1]]), d
    assert np.array_equal(S2, S[perm])


def test_chunk_fwd_is_deterministic():
    inp = kda_gen.make_prefill(31, 500, 4, "bf16", s0_std=0.02, s0_docs="all")
    o1, S1 = gpu_chunk_fwd(inp)
    o2, S2 = gpu_chunk_fwd(inp)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


@pytest.mark.parametrize("path", ["two_kernel", "fused", "fp32", "segment_scan", "unbounded",
                                  "decode", "decode_unbounded"])
def test_absent_A_log_is_zero(path):
    """A_log = NULL means A_h = 0 for every head: the same results, bit for bit,
    as an all-zero A_log, on the prefill paths and the decode step."""
    import linear_attention_fwd_amd as kda
    import torch
    from kda_testlib import gpu_inputs
    print(f"[case] A_log absent, path {path}", flush=True)
    if path.startswith("decode"):
        inp = kda_gen.make_decode(58, N=7, H=3, W=4, dtype="bf16", accepted=[0, 4, 2, 1, 3, 4, 0])
        unb = path == "decode_unbounded"
        outs = []
        for A in (torch.zeros(inp.H, dtype=torch.float32, device="cuda"), None):
            t = decode_gpu_inputs(inp)
            o = kda.kda_decode_step(t["state"], t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"],
                                    t["accepted"], t["nq"], t["nk"], t["nv"], t["nz"],
                                    t["nbeta"], A, inp.g_min, unbounded_gate=unb)
            torch.cuda.synchronize()
            outs.append((kda_gen.from_torch(o), kda_gen.from_torch(t["state"])))
    else:
        inp = kda_gen.make_prefill(38, 600, 3, "bf16", lengths=[300, 0, 299, 1], s0_std=0.02,
                                   s0_docs="all")
        t = gpu_inputs(inp)
        args = (t["q"], t["k"], t["v"], t["z"], t["beta"])
        compute = 1 if path == "fp32" else 0
        outs = []
        for A in (torch.zeros(inp.H, dtype=torch.float32, device="cuda"), None):
            if path == "segment_scan":
                o, S = kda.kda_segment_scan(*args, A, inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                            n_segments=4)
            else:
                o, S = kda.kda_chunk_fwd(*args, A, inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                         compute=compute, unbounded_gate=path == "unbounded",
                                         workspace=False if path == "fused" else None)
            torch.cuda.synchronize()
            outs.append((kda_gen.from_torch(o), kda_gen.from_torch(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("path", ["two_kernel", "fused", "fp32", "checkpoints", "noalloc",
                                  "segment_scan", "segment_scan_fp32"])
def test_prefill_without_final_state(path):
    """final_state = NULL (output_final_state=False) on every prefill path: O is
    the same bit for bit as with the final states written, nothing is written in
    their place (the documents include empty ones, whose final state would
    otherwise be a copy of the initial one)."""
    import linear_attention_fwd_amd as kda
    import torch
    from kda_testlib import gpu_inputs
    inp = kda_gen.make_prefill(37, 700, 3, "bf16", lengths=[130, 0, 257, 1, 0, 312],
                               s0_std=0.05, s0_docs="all")
    _case(inp, 1 if path.endswith("fp32") else 0)
    print(f"    path {path}", flush=True)
    t = gpu_inputs(inp)
    args = (t["q"], t["k"], t["v"], t["z"], t["beta"])
    compute = 1 if path.endswith("fp32") else 0

    def run(keep):
        if path == "checkpoints":
            return kda.kda_chunk_fwd_checkpoints(*args, 128, t["A_log"], inp.g_min, t["S0"],
                                                 t["cu"], t["cu_host"],
                                                 output_final_state=keep)[:2]
        if path == "noalloc":
            return kda.kda_chunk_fwd_noalloc(*args, t["A_log"], inp.g_min, t["S0"], t["cu"],
                                             t["cu_host"], output_final_state=keep)
        if path.startswith("segment_scan"):
            return kda.kda_segment_scan(*args, t["A_log"], inp.g_min, t["S0"], t["cu"],
                                        t["cu_host"], n_segments=5, output_final_state=keep,
                                        compute=compute)
        return kda.kda_chunk_fwd(*args, t["A_log"], inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                 output_final_state=keep, compute=compute,
                                 workspace=False if path == "fused" else None)

    o_ref, S_ref = run(True)
    o, S = run(False)
    torch.cuda.synchronize()
    assert S is None and S_ref is not None
    assert np.array_equal(kda_gen.from_torch(o), kda_gen.from_torch(o_ref))


@pytest.mark.parametrize("path", ["two_kernel", "fused", "fp32", "unbounded", "checkpoints"])
def test_final_state_in_place(path):
    """kda_chunk_fwd and its variants may write the final states over the initial
    states (each unit reads its initial state before it writes its final one):
    O and the states equal the out-of-place call bit for bit.  The documents
    include empty ones (final = initial, copied onto itself)."""
    import linear_attention_fwd_amd as kda
    import torch
    from kda_testlib import gpu_inputs
    inp = kda_gen.make_prefill(36, 700, 3, "bf16", lengths=[130, 0, 257, 1, 0, 312],
                               s0_std=0.05, s0_docs="all")
    _case(inp, 1 if path == "fp32" else 0)
    print(f"    path {path}", flush=True)
    t = gpu_inputs(inp)
    args = (t["q"], t["k"], t["v"], t["z"], t["beta"])

    def run(S_in, fin):
        if path == "unbounded":
            return kda.kda_chunk_fwd_unbounded(*args, t["A_log"], S_in, t["cu"], t["cu_host"],
                                               final_state=fin)[0]
        if path == "checkpoints":
            return kda.kda_chunk_fwd_checkpoints(*args, 128, t["A_log"], inp.g_min, S_in, t["cu"],
                                                 t["cu_host"], final_state=fin)[0]
        return kda.kda_chunk_fwd(*args, t["A_log"], inp.g_min, S_in, t["cu"], t["cu_host"],
                                 compute=1 if path == "fp32" else 0,
                                 workspace=False if path == "fused" else None, final_state=fin)[0]

    S_out = torch.empty_like(t["S0"])
    o_ref = kda_gen.from_torch(run(t["S0"], S_out))
    S_io = t["S0"].clone()
    o_in = kda_gen.from_torch(run(S_io, S_io))
    torch.cuda.synchronize()
    assert np.array_equal(o_in, o_ref)
    assert np.array_equal(kda_gen.from_torch(S_io), kda_gen.from_torch(S_out))
    assert np.array_equal(kda_gen.from_torch(S_io)[[1, 4]], inp.S0[[1, 4]])


def test_chunk_fwd_resume_equals_one_call():
    """Splitting a document at a chunk-aligned token and carrying the final
    state gives the one-call result (the chunking is then identical)."""
    inp = kda_gen.make_prefill(32, 384, 2, "bf16", s0_std=0.02, s0_docs="all")
    o_all, S_all = gpu_chunk_fwd(inp)
    cut = 192
    a = kda_gen.PrefillInputs(*(kda_gen.Tensor(x.data[:cut], x.dtype) for x in
                                (inp.q, inp.k, inp.v, inp.z, inp.beta)), inp.A_log, inp.S0,
                              np.array([0, cut], np.int32), inp.g_min, inp.dtype)
    oa, Sa = gpu_chunk_fwd(a)
    b = kda_gen.PrefillInputs(*(kda_gen.Tensor(x.data[cut:], x.dtype) for x in
                                (inp.q, inp.k, inp.v, inp.z, inp.beta)), inp.A_log,
                              Sa.astype(np.float32), np.array([0, inp.T - cut], np.int32),
                              inp.g_min, inp.dtype)
    ob, Sb = gpu_chunk_fwd(b)
    assert np.array_equal(np.concatenate([oa, ob]), o_all)
    assert np.array_equal(Sb, S_all)


def _units_fill_device(units):
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"    (document|segment, head) units {units}, compute units {cus}: "
          f"{'two' if units >= cus else 'one'} column tile(s) per compute wave", flush=True)


def test_many_documents_wide_recurrence():
    """Enough (document, head) units to fill the device: the recurrence runs
    128 columns per workgroup.  Against the oracle and the fused kernel."""
    rng = np.random.default_rng(35)
    lengths = [int(x) for x in rng.integers(0, 150, size=40)] + [0, 1, 64, 65]
    inp = kda_gen.make_prefill(35, int(sum(lengths)), 8, "bf16", lengths=lengths, s0_std=0.02,
                               s0_docs="all")
    _case(inp, 0)
    _units_fill_device(inp.N * inp.H)
    o, S = gpu_chunk_fwd(inp)
    _check_prefill(inp, o, S, _tols(inp, 0))
    o2, S2 = gpu_chunk_fwd(inp, fused=True)
    eo, _ = rel_l2_slices(o, o2, inp.cu_seqlens)
    es, _ = rel_l2_slices(S, S2, axis_tokens=False)
    print(f"    vs fused kernel: O {eo:.3e} S {es:.3e}", flush=True)
    assert eo <= 1e-3 and es <= 1e-3, (eo, es)


def test_segment_scan_many_segments_wide_recurrence():
    """Segment pairs and re-runs with 128 columns per workgroup (enough
    (segment, head) units to fill the device), segments of one chunk slot."""
    inp = kda_gen.make_prefill(45, 4100, 8, "bf16", lengths=[1000, 64, 0, 2500, 536],
                               s0_std=0.05, s0_docs="all")
    _case(inp, 0)
    print("    n_segments=256", flush=True)
    _units_fill_device(69 * inp.H)  # 4100 // 64 + 5 chunk slots, one per segment
    o, S = gpu_segment_scan(inp, n_segments=256)
    _check_prefill(inp, o, S, _tols(inp, 0))


def test_segment_scan_wide_compose():
    """A compose of 8 groups x 32 heads = 256 chains over 256 columns: enough for
    64-column slices at four per compute unit (the widest shape of the chain
    kernel); 64 segments of one chunk slot, a ragged last document."""
    import linear_attention_fwd_amd as kda
    inp = kda_gen.make_prefill(50, 4096 - 37, 32, "bf16", lengths=[1500, 2559], s0_std=0.05,
                               s0_docs="all")
    _case(inp, 0)
    n_cu = kda.kda_default_segments()
    print(f"    n_segments=64 ({n_cu} compute units)", flush=True)
    if 8 * inp.H * 4 < 4 * n_cu:
        pytest.skip("this device needs more chains for the widest compose shape")
    o, S = gpu_segment_scan(inp, n_segments=64)
    _check_prefill(inp, o, S, _tols(inp, 0))


CHECKPOINT_CASES = {
    # name: (generator kwargs, interval in tokens)
    "varlen_128": (dict(seed=47, T=2300, H=3, dtype="bf16", lengths=[700, 0, 129, 1024, 383, 64],
                        s0_std=0.02, s0_docs="all"), 128),
    "single_doc_512": (dict(seed=48, T=2048, H=2, dtype="bf16", z_mean=-6.0, s0_std=0.05,
                            s0_docs="all"), 512),
    # every chunk boundary, raw inputs (normalised in the prep kernel)
    "every_chunk_raw_64": (dict(seed=68, T=900, H=2, dtype="bf16", lengths=[64, 65, 771],
                                s0_std=0.05, s0_docs="all", raw=True), 64),
}


@pytest.mark.parametrize("name", sorted(CHECKPOINT_CASES))
def test_checkpoints_match_oracle(name):
    """States emitted every `interval` tokens inside each document equal the
    oracle's state after that prefix; O and the final states are those of
    kda_chunk_fwd, bit for bit."""
    import linear_attention_fwd_amd as kda
    import torch
    from kda_testlib import gpu_inputs, oracle_checkpoints
    kw, interval = CHECKPOINT_CASES[name]
    kw = dict(kw)
    seed, T, H = kw.pop("seed"), kw.pop("T"), kw.pop("H")
    inp = kda_gen.make_prefill(seed, T, H, **kw)
    _case(inp, 0)
    print(f"    checkpoint interval {interval}", flush=True)
    t = gpu_inputs(inp)
    o1, S1 = gpu_chunk_fwd(inp, t=t)
    o2, S2, ck = kda.kda_chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["z"], t["beta"], interval,
                                               t["A_log"], inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                               raw_inputs=inp.raw)
    torch.cuda.synchronize()
    assert np.array_equal(o1, kda_gen.from_torch(o2)) and np.array_equal(S1, kda_gen.from_torch(S2))
    ck = kda_gen.from_torch(ck)
    ref = oracle_checkpoints(inp, interval)
    assert ref, "the case must have checkpoints"
    worst = 0.0
    for (d, j), S_ref in ref.items():
        i = kda.checkpoint_index(inp.cu_seqlens, d, j, interval)
        for hh in range(inp.H):
            e = np.linalg.norm(ck[i, hh] - S_ref[hh]) / np.linalg.norm(S_ref[hh])
            worst = max(worst, e)
    print(f"    {len(ref)} checkpoints, max rel L2 {worst:.3e}", flush=True)
    assert worst <= TOL_BF16, worst


def test_checkpoints_wide_recurrence():
    """Checkpoints from the 128-column recurrence (enough documents to fill the
    device)."""
    import linear_attention_fwd_amd as kda
    import torch
    from kda_testlib import gpu_inputs, oracle_checkpoints
    rng = np.random.default_rng(49)
    lengths = [int(x) for x in rng.integers(0, 400, size=36)]
    interval = 192
    inp = kda_gen.make_prefill(49, int(sum(lengths)), 8, "bf16", lengths=lengths, s0_std=0.02,
                               s0_docs="all")
    _case(inp, 0)
    _units_fill_device(inp.N * inp.H)
    t = gpu_inputs(inp)
    o, S, ck = kda.kda_chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["z"], t["beta"], interval,
                                             t["A_log"], inp.g_min, t["S0"], t["cu"], t["cu_host"])
    torch.cuda.synchronize()
    _check_prefill(inp, kda_gen.from_torch(o), kda_gen.from_torch(S), _tols(inp, 0))
    ck = kda_gen.from_torch(ck)
    ref = oracle_checkpoints(inp, interval)
    worst = max(np.linalg.norm(ck[kda.checkpoint_index(inp.cu_seqlens, d, j, interval), hh] - S_ref[hh])
                / np.linalg.norm(S_ref[hh]) for (d, j), S_ref in ref.items() for hh in range(inp.H))
    print(f"    {len(ref)} checkpoints, max rel L2 {worst:.3e}", flush=True)
    assert worst <= TOL_BF16, worst


SCAN_CASES = {
    # lengths chosen so that segment boundaries fall inside documents, exactly on
    # a document start (n_seg=7 -> segments of 215 tokens; a document starts at 430),
    # and segments contain several document starts
    "varlen_bf16": dict(seed=41, T=1505, H=2, dtype="bf16",
                        lengths=[100, 330, 0, 700, 3, 2, 370], s0_std=0.05, s0_docs="all"),
    "single_doc_fp32": dict(seed=42, T=900, H=2, dtype="f32", s0_std=0.1, s0_docs="all"),
    "slow_decay_single_doc": dict(seed=43, T=1300, H=2, dtype="bf16", z_mean=-6.0,
                                  s0_std=0.05, s0_docs="all"),
}


@pytest.mark.parametrize("name", sorted(SCAN_CASES))
@pytest.mark.parametrize("n_seg", [0, 1, 7, 64])
def test_segment_scan_matches_oracle(name, n_seg):
    kw = dict(SCAN_CASES[name])
    seed, T, H = kw.pop("seed"), kw.pop("T"), kw.pop("H")
    inp = kda_gen.make_prefill(seed, T, H, **kw)
    ref = oracle_forward(inp)
    for compute in ((0,) if inp.dtype == "f32" else (0, 1)):
        _case(inp, compute)
        print(f"    n_segments={n_seg}", flush=True)
        o, S = gpu_segment_scan(inp, n_segments=n_seg, compute=compute)
        _check_prefill(inp, o, S, _tols(inp, compute), ref)


DEFAULT_PLAN_CASES = {
    # n_segments = 0 with H >= CUs / 32: ceil(CUs / H) segments per head, each its
    # own group, scanned in one level.  Document d's first chunk slot is
    # floor(cu[d] / 64) + d.  At 256 CUs: H=8 asks for 32 segments over 46 used
    # slots -> 23 segments of 2 slots, documents starting on segment boundaries
    # (slots 12, 32, 34) and inside one (slot 15), an empty document between;
    # H=12 asks for 22 -> 16 segments of 3 slots (long memory); H=40 asks for 7
    # -> 7 of 5 slots, a one-token document on a boundary (slot 15) and the next
    # document inside a segment (slot 16); H=96 asks for 3 -> 3 of 4 slots.
    "h8_varlen": dict(seed=71, T=2600, H=8, dtype="bf16", lengths=[704, 100, 0, 1000, 64, 732],
                      s0_std=0.05, s0_docs="all"),
    "h12_slow_decay": dict(seed=72, T=3000, H=12, dtype="bf16", z_mean=-6.0, s0_std=0.05,
                           s0_docs="all"),
    "h40_varlen": dict(seed=73, T=1800, H=40, dtype="bf16", lengths=[900, 1, 899],
                       s0_std=0.05, s0_docs="all"),
    "h96_single": dict(seed=74, T=700, H=96, dtype="bf16", s0_std=0.05, s0_docs="all"),
    # the same plan with the unbounded gate (strong decays) and on raw inputs
    "h8_unbounded": dict(seed=75, T=2000, H=8, dtype="bf16", lengths=[1100, 0, 900],
                         gate="softplus", z_mean=2.0, z_std=3.0, A_std=1.0, s0_std=0.05,
                         s0_docs="all"),
    "h8_raw": dict(seed=76, T=2000, H=8, dtype="bf16", lengths=[640, 1360], raw=True,
                   s0_std=0.05, s0_docs="all"),
}


@pytest.mark.parametrize("name", sorted(DEFAULT_PLAN_CASES))
def test_segment_scan_default_plan(name):
    """The default segment plan (one (segment, head) per compute unit, one level)
    against the oracle, with bf16 and fp32 arithmetic."""
    kw = dict(DEFAULT_PLAN_CASES[name])
    seed, T, H = kw.pop("seed"), kw.pop("T"), kw.pop("H")
    inp = kda_gen.make_prefill(seed, T, H, **kw)
    ref = oracle_forward(inp)
    # raw bf16 inputs take bf16 arithmetic only (fp32 arithmetic on them is refused)
    for compute in ((0,) if inp.raw else (0, 1)):
        _case(inp, compute)
        print("    n_segments=0", flush=True)
        o, S = gpu_segment_scan(inp, n_segments=0, compute=compute)
        _check_prefill(inp, o, S, _tols(inp, compute), ref)


def test_segment_scan_one_segment_equals_chunk_fwd():
    """One segment re-runs every chunk from the start: with bf16 arithmetic the
    recurrence kernel of the two-kernel chunk_fwd, with fp32 arithmetic the fused
    kernel, in both cases bit for bit."""
    inp = kda_gen.make_prefill(44, 640, 2, "bf16", lengths=[200, 440], s0_std=0.02,
                               s0_docs="all")
    o1, S1 = gpu_chunk_fwd(inp)
    o2, S2 = gpu_segment_scan(inp, n_segments=1)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    o1, S1 = gpu_chunk_fwd(inp, compute=1)
    o2, S2 = gpu_segment_scan(inp, n_segments=1, compute=1)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ---------------------------------------------------------------------------
# the unbounded (softplus) gate: per-position diagonal subtiles
# ---------------------------------------------------------------------------
UNBOUNDED_CASES = {
    # ordinary logits: decays of the same order as the bounded gate's
    "single_ragged_1000": dict(seed=61, T=1000, H=4),
    # strong decays (per-step log-decay down to about -100): a 16-token subtile
    # spans far more than the fp32 exponent range, so only the per-position path
    # can form its diagonal block; documents with initial states, a ragged tail
    "strong_decay_varlen": dict(seed=62, T=1500, H=4, lengths=[700, 13, 64, 723], z_mean=2.0,
                                z_std=3.0, A_std=1.0, s0_std=0.05, s0_docs="all"),
    # about -5.2 per step: the diagonal subtiles' decay ranges straddle the
    # limit of the two-factor MFMA form (116 in base 2, beyond the bounded
    # gate's 108), so it runs right at its edge, beside per-position subtiles
    # in the same chunks
    "two_factor_limit": dict(seed=64, T=640, H=4, z_mean=5.15, z_std=0.3, A_std=0.0),
}


@pytest.mark.parametrize("path", ["two_kernel", "fused", "fp32"])
def test_unbounded_gate_single_token_and_empty_document(path):
    """The unbounded gate on a one-token document beside an empty one and a
    ragged 70-token one, on each prefill path (fp32: fp32 inputs): partial chunks
    pad with zeros, the empty document passes its initial state through."""
    dtype = "f32" if path == "fp32" else "bf16"
    inp = kda_gen.make_prefill(63, 71, 2, dtype, lengths=[1, 0, 70], s0_std=0.05,
                               s0_docs="all", gate="softplus")
    _case(inp, 0)
    print(f"    path {path}", flush=True)
    o, S = gpu_chunk_fwd_unbounded(inp, fused=path == "fused")
    _check_prefill(inp, o, S, _tols(inp, 0))
    assert np.array_equal(S[1], inp.S0[1])


def test_all_documents_empty():
    """T = 0: nothing to run, every final state is the document's initial state
    (chunk kernels, segment scan and the unbounded gate, bf16 and fp32 inputs,
    with and without a workspace)."""
    import torch
    import linear_attention_fwd_amd as kda
    H = 2
    S0 = np.random.default_rng(67).standard_normal((3, H, 128, 128)).astype(np.float32)
    z = torch.zeros((0, H, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    zf, bf = z.float(), b.float()
    s0 = torch.from_numpy(S0).cuda()
    cu_host = np.zeros(4, dtype=np.int32)
    cu = torch.from_numpy(cu_host).cuda()
    print("[case] T=0, 3 empty documents", flush=True)
    for name, call in (
            ("chunk_fwd", lambda: kda.kda_chunk_fwd(z, z, z, z, b, None, -5.0, s0, cu, cu_host)),
            ("chunk_fwd fused", lambda: kda.kda_chunk_fwd(z, z, z, z, b, None, -5.0, s0, cu, cu_host,
                                                          workspace=False)),
            ("chunk_fwd fp32", lambda: kda.kda_chunk_fwd(zf, zf, zf, zf, bf, None, -5.0, s0, cu,
                                                         cu_host)),
            ("segment_scan", lambda: kda.kda_segment_scan(z, z, z, z, b, None, -5.0, s0, cu, cu_host,
                                                          n_segments=4)),
            ("segment_scan fp32", lambda: kda.kda_segment_scan(zf, zf, zf, zf, bf, None, -5.0, s0, cu,
                                                               cu_host, n_segments=4)),
            ("unbounded", lambda: kda.kda_chunk_fwd_unbounded(z, z, z, z, b, None, s0, cu, cu_host)),
            ("unbounded fused", lambda: kda.kda_chunk_fwd_unbounded(z, z, z, z, b, None, s0, cu, cu_host,
                                                                    workspace=False)),
            ("unbounded fp32", lambda: kda.kda_chunk_fwd_unbounded(zf, zf, zf, zf, bf, None, s0, cu,
                                                                   cu_host))):
        print(f"    {name}", flush=True)
        o, S = call()
        torch.cuda.synchronize()
        assert o.shape == (0, H, 128)
        assert np.array_equal(kda_gen.from_torch(S), S0), name


def _diagonal_subtile_forms(inp):
    """(subtile-heads whose decay range G_s - G_e stays within 116 in base 2
    in every channel, those beyond it), from the oracle's gate: the kernels
    form the first kind's diagonal block with two MFMA factors, the second
    per position."""
    g = oracle.gate_softplus(inp.z.f64(), inp.A_log)
    cu = inp.cu_seqlens
    within = beyond = 0
    for d in range(inp.N):
        for c0 in range(cu[d], cu[d + 1], 64):
            for s0 in range(c0, min(c0 + 64, cu[d + 1]), 16):
                decay = -g[s0 + 1:min(s0 + 16, cu[d + 1])].sum(axis=0) / np.log(2.0)
                ok = (decay <= 116.0).all(axis=-1)
                within += int(ok.sum())
                beyond += int((~ok).sum())
    return within, beyond


@pytest.mark.parametrize("path", ["two_kernel", "fused", "fp32"])
@pytest.mark.parametrize("name", sorted(UNBOUNDED_CASES))
def test_unbounded_gate_matches_oracle(name, path):
    """The unbounded gate on the bf16 two-kernel path and the bf16 fused kernel
    (1e-2), and on fp32 inputs through the fp32 verification build (1e-4), which
    forms the same two-factor and per-position diagonal subtiles in fp32."""
    c = dict(UNBOUNDED_CASES[name])
    seed, T, H = c.pop("seed"), c.pop("T"), c.pop("H")
    dtype = "f32" if path == "fp32" else "bf16"
    inp = kda_gen.make_prefill(seed, T, H, dtype, gate="softplus", **c)
    print(f"[case] unbounded gate {name} T={T} H={H} N={inp.N} path {path}", flush=True)
    within, beyond = _diagonal_subtile_forms(inp)
    print(f"    diagonal subtile-heads: {within} two-factor, {beyond} per position", flush=True)
    if name == "strong_decay_varlen":
        G = np.cumsum(oracle.gate_softplus(inp.z.f64()[:16], inp.A_log), axis=0)
        assert (G[0] - G[15]).max() > 100.0  # e^100 is beyond fp32
    assert within > 0 and (beyond > 0) == (name != "single_ragged_1000")
    o_ref, S_ref = oracle_forward(inp)
    o, S = gpu_chunk_fwd_unbounded(inp, fused=path == "fused")
    assert np.isfinite(o).all() and np.isfinite(S).all()
    eo, _ = rel_l2_slices(o, o_ref, inp.cu_seqlens)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"    o: {eo:.3e}  state: {es:.3e}", flush=True)
    tol = TOL_F32 if path == "fp32" else TOL_BF16
    assert eo <= tol and es <= tol
    if path == "fused":  # the same stages as the two kernels
        o2, S2 = gpu_chunk_fwd_unbounded(inp)
        print(f"    identical to the two-kernel path: O {np.array_equal(o, o2)}, "
              f"S {np.array_equal(S, S2)}", flush=True)
        eo2, _ = rel_l2_slices(o, o2, inp.cu_seqlens)
        es2, _ = rel_l2_slices(S, S2, axis_tokens=False)
        assert eo2 <= 1e-3 and es2 <= 1e-3, (eo2, es2)


@pytest.mark.parametrize("path", ["chunk_fwd_flag", "segment_scan", "segment_scan_fp32",
                                  "checkpoints", "noalloc", "prep_recurrence"])
def test_unbounded_gate_other_entry_points(path):
    """KDA_UNBOUNDED_GATE on the prefill entry points besides kda_chunk_fwd_unbounded:
    the segment scan (two kernels, and fp32 inputs through the fused kernel), the
    checkpoint prefill (checked against the oracle's state after each prefix too),
    the no-allocation call and the two halves called on their own (both bit for
    bit equal to kda_chunk_fwd_unbounded), on strong decays with both diagonal
    forms, documents with initial states and a ragged tail.  g_min is passed as
    -7, which the bounded gate would refuse: the unbounded gate does not use it."""
    import dataclasses
    import torch
    import linear_attention_fwd_amd as kda
    from kda_testlib import gpu_inputs, oracle_checkpoints
    c = dict(UNBOUNDED_CASES["strong_decay_varlen"])
    seed, T, H = c.pop("seed"), c.pop("T"), c.pop("H")
    dtype = "f32" if path.endswith("fp32") else "bf16"
    inp = kda_gen.make_prefill(seed, T, H, dtype, gate="softplus", **c)
    inp = dataclasses.replace(inp, g_min=-7.0)
    print(f"[case] unbounded gate via the flag, {path}, T={T} H={H} N={inp.N}", flush=True)
    t = gpu_inputs(inp)
    ref = gpu_chunk_fwd_unbounded(dataclasses.replace(inp, g_min=-5.0), t=t)
    if path == "chunk_fwd_flag":
        o, S = gpu_chunk_fwd(inp, t=t)
        assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1])
    elif path.startswith("segment_scan"):
        o, S = gpu_segment_scan(inp, n_segments=7, t=t)
    elif path == "checkpoints":
        interval = 128
        o, S, ck = kda.kda_chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["z"], t["beta"],
                                                 interval, t["A_log"], inp.g_min, t["S0"], t["cu"],
                                                 t["cu_host"], unbounded_gate=True)
        torch.cuda.synchronize()
        o, S, ck = kda_gen.from_torch(o), kda_gen.from_torch(S), kda_gen.from_torch(ck)
        assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1])
        want = oracle_checkpoints(inp, interval)
        worst = 0.0
        for (d, j), Sref in want.items():
            i = kda.checkpoint_index(inp.cu_seqlens, d, j, interval)
            e, _ = rel_l2_slices(ck[i][None], Sref[None], axis_tokens=False)
            worst = max(worst, e)
        print(f"    {len(want)} checkpoints, worst state {worst:.3e}", flush=True)
        assert worst <= TOL_BF16
    elif path == "noalloc":
        o, S = kda.kda_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"],
                                         inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                         unbounded_gate=True)
        torch.cuda.synchronize()
        o, S = kda_gen.from_torch(o), kda_gen.from_torch(S)
        assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1])
    else:
        ws = torch.empty(kda.kda_chunk_fwd_workspace_size(inp.N, T, H), dtype=torch.uint8,
                         device="cuda")
        kda.kda_chunk_prep(t["q"], t["k"], t["z"], t["beta"], ws, t["A_log"], inp.g_min,
                           t["cu"], t["cu_host"], unbounded_gate=True)
        o, S = kda.kda_chunk_recurrence(t["v"], ws, t["S0"], t["cu"], t["cu_host"])
        torch.cuda.synchronize()
        o, S = kda_gen.from_torch(o), kda_gen.from_torch(S)
        assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1])
    _check_prefill(inp, o, S, _tols(inp, 0))


# ---------------------------------------------------------------------------
# raw inputs: q, k normalised and beta = sigmoid(logit) in the kernels
# ---------------------------------------------------------------------------
def _zero_rows(t, rows):
    t.data[rows] = 0
    return t


@pytest.mark.parametrize("path", ["chunk_fwd", "segment_scan", "unbounded", "fused",
                                  "unbounded_fused", "fp32", "segment_scan_fp32",
                                  "unbounded_fp32"])
def test_raw_inputs_prefill(path):
    """Unnormalised q, k and beta logits through the two-kernel prefill (and the
    segment scan and the unbounded gate, which share its prep), the fused kernel
    (bf16), and the fp32 verification build on fp32 inputs (1e-4; documents and
    segments), against the oracle that normalises them.  Some tokens have all-zero q or k rows (their
    normalised rows stay zero)."""
    dtype = "f32" if path.endswith("fp32") else "bf16"
    inp = kda_gen.make_prefill(64, 1200, 4, dtype, lengths=[500, 0, 77, 623], s0_std=0.05,
                               s0_docs="all", raw=True,
                               gate="softplus" if path.startswith("unbounded") else "bounded")
    _zero_rows(inp.q, [3, 600, 1199])
    _zero_rows(inp.k, [4, 577, 1000])
    _case(inp, 0)
    print(f"    raw inputs, {path}", flush=True)
    o_ref, S_ref = oracle_forward(inp)
    if path in ("chunk_fwd", "fused", "fp32"):
        o, S = gpu_chunk_fwd(inp, fused=path == "fused")
    elif path.startswith("segment_scan"):
        o, S = gpu_segment_scan(inp, n_segments=7)
    else:
        o, S = gpu_chunk_fwd_unbounded(inp, fused=path == "unbounded_fused")
    assert np.all(o[[3, 600, 1199]] == 0)
    _check_prefill(inp, o, S, _tols(inp, 0))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_raw_inputs_decode_window(dtype):
    """Raw draft, bonus and next-window inputs through the decode kernel."""
    inp = kda_gen.make_decode(65, N=24, H=4, W=4, dtype=dtype,
                              accepted=[i % 5 for i in range(24)], W2=3, raw=True)
    print(f"[case] raw decode window N={inp.N} H={inp.H} dtype={dtype}", flush=True)
    o_ref, ow_ref, S_ref = oracle.decode_window(inp)
    o, ow, S = gpu_decode_window(inp)
    o1, S1 = gpu_decode(inp)
    assert np.array_equal(o, o1) and np.array_equal(S, S1)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    ew = max(rel_l2_slices(ow[:, j][:, :, None], ow_ref[:, j][:, :, None], axis_tokens=False)[0]
             for j in range(3))
    print(f"    o: {eo:.3e}  window: {ew:.3e}  state: {es:.3e}", flush=True)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert eo <= tol and ew <= tol and es <= tol


# ---------------------------------------------------------------------------
# decode with speculative-verify replay
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["bounded", "softplus"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_matches_oracle(dtype, gate):
    """Replay + bonus from the saved state; with gate="softplus" the unbounded gate
    (KDA_UNBOUNDED_GATE) that a model prefilled with it decodes with."""
    inp = kda_gen.make_decode(51, N=40, H=4, W=4, dtype=dtype,
                              accepted=[i % 5 for i in range(40)], gate=gate)
    print(f"[case] decode N={inp.N} H={inp.H} W={inp.W} dtype={dtype} gate={gate}", flush=True)
    o_ref, S_ref = oracle.decode(inp)
    o, S = gpu_decode(inp)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    print(f"    o: {eo:.3e}  state: {es:.3e}", flush=True)
    # fp32 arithmetic throughout: the state matches to fp32 accuracy; o is stored
    # in the input dtype (bf16 rounding alone is ~2e-3 relative)
    assert es <= TOL_F32
    assert eo <= (TOL_F32 if dtype == "f32" else TOL_BF16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_long_draft_cache(dtype):
    """A draft cache of W = 12: replays of up to 13 tokens span two staging
    batches of 8, so the bonus token and the state kept fall in the second batch
    for some sequences and in the first for others; a next window of 3 drafts
    follows on either side of that boundary."""
    accepted = [0, 1, 5, 6, 7, 8, 9, 11, 12, 12, 3, 10]
    inp = kda_gen.make_decode(57, N=len(accepted), H=3, W=12, dtype=dtype, accepted=accepted,
                              W2=3)
    print(f"[case] decode long cache N={inp.N} H={inp.H} W={inp.W} W2=3 dtype={dtype}",
          flush=True)
    o_ref, S_ref = oracle.decode(inp)
    _, ow_ref, _ = oracle.decode_window(inp)
    o, S = gpu_decode(inp)
    o2, ow, S2 = gpu_decode_window(inp)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    ew = max(rel_l2_slices(ow[:, j][:, :, None], ow_ref[:, j][:, :, None], axis_tokens=False)[0]
             for j in range(3))
    print(f"    o: {eo:.3e}  window: {ew:.3e}  state: {es:.3e}", flush=True)
    assert es <= TOL_F32
    assert eo <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    assert ew <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_decode_slots_and_clamping():
    import torch
    inp = kda_gen.make_decode(52, N=6, H=2, W=4, dtype="bf16", accepted=[0, 4, 7, -1, 2, 3])
    t = decode_gpu_inputs(inp)
    # a state pool twice as large, sequences scattered into it
    slots = np.array([9, 0, 4, 11, 6, 2], dtype=np.int32)
    pool = np.zeros((12, inp.H, 128, 128), np.float32)
    pool[slots] = inp.state
    t["state"] = torch.from_numpy(pool).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, P = gpu_decode(inp, t=t, state_slots=torch.from_numpy(slots).cuda(), err_flag=err)
    assert int(err.item()) == 1  # 7 and -1 were out of range
    clamped = kda_gen.make_decode(52, N=6, H=2, W=4, dtype="bf16", accepted=[0, 4, 4, 0, 2, 3])
    o_ref, S_ref = oracle.decode(clamped)
    es, _ = rel_l2_slices(P[slots], S_ref, axis_tokens=False)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    assert es <= TOL_F32 and eo <= TOL_BF16
    untouched = np.setdiff1d(np.arange(12), slots)
    assert np.all(P[untouched] == 0)


@pytest.mark.parametrize("W2", [0, 3])
def test_decode_skips_slots_outside_the_pool(W2):
    """Slots -1 and S_pool (a padding convention and an off-by-one) are skipped:
    the pool is neither read nor written there, those sequences' outputs are
    zeros, err_flag gets the slot bit, and every other sequence is unaffected."""
    import torch
    import linear_attention_fwd_amd as kda
    inp = kda_gen.make_decode(56, N=6, H=2, W=4, dtype="bf16", accepted=[1, 4, 0, 3, 2, 4], W2=W2)
    S_pool = 8
    slots = np.array([5, -1, 0, S_pool, 7, 2], dtype=np.int32)
    good = slots >= 0
    pool = np.full((S_pool, inp.H, 128, 128), 3.0, np.float32)  # sentinel for unused slots
    pool[slots[good & (slots < S_pool)]] = inp.state[good & (slots < S_pool)]
    print(f"[case] decode with slots {slots.tolist()} in a pool of {S_pool}, W2={W2}", flush=True)
    t = decode_gpu_inputs(inp)
    t["state"] = torch.from_numpy(pool).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sl = torch.from_numpy(slots).cuda()
    if W2:
        o, ow, P = gpu_decode_window(inp, t=t, state_slots=sl, err_flag=err)
        _, ow_ref, _ = oracle.decode_window(inp)
    else:
        o, P = gpu_decode(inp, t=t, state_slots=sl, err_flag=err)
    assert int(err.item()) == kda.KDA_DECODE_ERR_SLOT
    bad = ~((slots >= 0) & (slots < S_pool))
    assert np.all(o[bad] == 0)
    o_ref, S_ref = oracle.decode(inp)
    ok = ~bad
    assert rel_l2_slices(P[slots[ok]], S_ref[ok], axis_tokens=False)[0] <= TOL_F32
    assert rel_l2_slices(o[ok][:, :, None], o_ref[ok][:, :, None], axis_tokens=False)[0] <= TOL_BF16
    if W2:
        assert np.all(ow[bad] == 0)
        assert rel_l2_slices(ow[ok].reshape(-1, inp.H, 128)[:, :, None],
                             ow_ref[ok].reshape(-1, inp.H, 128)[:, :, None],
                             axis_tokens=False)[0] <= TOL_BF16
    untouched = np.setdiff1d(np.arange(S_pool), slots[ok])
    assert np.all(P[untouched] == 3.0)


@pytest.mark.parametrize("dtype,W2,gate", [("bf16", 4, "bounded"), ("f32", 4, "bounded"),
                                           ("bf16", 13, "bounded"), ("f32", 1, "bounded"),
                                           ("f32", 7, "bounded"), ("bf16", 4, "softplus"),
                                           ("f32", 7, "softplus")])
def test_decode_window_matches_oracle(dtype, W2, gate):
    """Replay + bonus + next draft window in one kernel: the bonus output and the
    state kept equal those of kda_decode_step bit for bit (the same arithmetic on
    the same tokens), and the window drafts' outputs match the oracle.  The last
    draft of a window takes its own path (no state update): W2 = 1 makes it the
    only draft, W2 = 7 puts it in the first staging batch or the second depending
    on the accepted length, W2 = 13 runs the token loop past two batches."""
    import torch
    inp = kda_gen.make_decode(54, N=24, H=4, W=4, dtype=dtype,
                              accepted=[i % 5 for i in range(24)], W2=W2, gate=gate)
    print(f"[case] decode window N={inp.N} H={inp.H} W={inp.W} W2={W2} dtype={dtype} "
          f"gate={gate}", flush=True)
    o_ref, ow_ref, S_ref = oracle.decode_window(inp)
    o, ow, S = gpu_decode_window(inp)
    o1, S1 = gpu_decode(inp)
    assert np.array_equal(S, S1)
    assert np.array_equal(o, o1)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    ew = max(rel_l2_slices(ow[:, j][:, :, None], ow_ref[:, j][:, :, None], axis_tokens=False)[0]
             for j in range(W2))
    print(f"    o: {eo:.3e}  window: {ew:.3e}  state: {es:.3e}", flush=True)
    assert es <= TOL_F32
    assert eo <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    assert ew <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_decode_window_slots_and_empty_window():
    """Pool slots with the window; W2 = 0 is the plain decode step."""
    import torch
    import linear_attention_fwd_amd as kda
    inp = kda_gen.make_decode(55, N=6, H=2, W=4, dtype="bf16", accepted=[0, 4, 1, 3, 2, 4], W2=2)
    slots = np.array([7, 0, 3, 10, 5, 1], dtype=np.int32)
    pool = np.zeros((11, inp.H, 128, 128), np.float32)
    pool[slots] = inp.state
    t = decode_gpu_inputs(inp)
    t["state"] = torch.from_numpy(pool).cuda()
    o, ow, P = gpu_decode_window(inp, t=t, state_slots=torch.from_numpy(slots).cuda())
    o_ref, ow_ref, S_ref = oracle.decode_window(inp)
    assert rel_l2_slices(P[slots], S_ref, axis_tokens=False)[0] <= TOL_F32
    assert rel_l2_slices(ow.reshape(-1, inp.H, 128)[:, :, None],
                         ow_ref.reshape(-1, inp.H, 128)[:, :, None], axis_tokens=False)[0] <= TOL_BF16
    untouched = np.setdiff1d(np.arange(11), slots)
    assert np.all(P[untouched] == 0)
    # an empty window
    t0 = decode_gpu_inputs(inp)
    e = torch.empty((inp.N, 0, inp.H, 128), dtype=t0["wq"].dtype, device="cuda")
    eb = torch.empty((inp.N, 0, inp.H), dtype=t0["wq"].dtype, device="cuda")
    o0, ow0 = kda.kda_decode_step_window(
        t0["state"], t0["cq"], t0["ck"], t0["cv"], t0["cz"], t0["cbeta"], t0["accepted"],
        t0["nq"], t0["nk"], t0["nv"], t0["nz"], t0["nbeta"], e, e, e, e, eb, t0["A_log"],
        inp.g_min)
    torch.cuda.synchronize()
    o1, S1 = gpu_decode(inp)
    assert ow0.shape == (inp.N, 0, inp.H, 128)
    assert np.array_equal(kda_gen.from_torch(o0), o1)
    assert np.array_equal(kda_gen.from_torch(t0["state"]), S1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_without_drafts(dtype):
    """W = 0: no draft cache at all, the step is the bonus token alone (with and
    without a next window)."""
    inp = kda_gen.make_decode(66, N=9, H=3, W=0, dtype=dtype, W2=2)
    print(f"[case] decode without drafts N={inp.N} H={inp.H} dtype={dtype}", flush=True)
    o_ref, S_ref = oracle.decode(inp)
    o, S = gpu_decode(inp)
    eo, _ = rel_l2_slices(o[:, :, None], o_ref[:, :, None], axis_tokens=False)
    es, _ = rel_l2_slices(S, S_ref, axis_tokens=False)
    assert es <= TOL_F32 and eo <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    _, ow_ref, _ = oracle.decode_window(inp)
    o2, ow, S2 = gpu_decode_window(inp)
    assert np.array_equal(o2, o) and np.array_equal(S2, S)
    ew = max(rel_l2_slices(ow[:, j][:, :, None], ow_ref[:, j][:, :, None], axis_tokens=False)[0]
             for j in range(2))
    assert ew <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_decode_equals_chunk_fwd_on_the_same_tokens():
    """A replay of a accepted drafts + bonus equals a prefill over those a+1 tokens
    from the saved state (two independent GPU paths)."""
    inp = kda_gen.make_decode(53, N=5, H=2, W=4, dtype="f32", accepted=[4, 4, 4, 4, 4])
    o_dec, S_dec = gpu_decode(inp)
    n = 3
    toks = lambda c, nb: np.concatenate([c.data[n], nb.data[n][None]])
    pre = kda_gen.PrefillInputs(
        kda_gen.Tensor(toks(inp.cq, inp.nq), "f32"), kda_gen.Tensor(toks(inp.ck, inp.nk), "f32"),
        kda_gen.Tensor(toks(inp.cv, inp.nv), "f32"), kda_gen.Tensor(toks(inp.cz, inp.nz), "f32"),
        kda_gen.Tensor(np.concatenate([inp.cbeta.data[n], inp.nbeta.data[n][None]]), "f32"),
        inp.A_log, inp.state[n:n + 1], np.array([0, 5], np.int32), inp.g_min, "f32")
    o_pre, S_pre = gpu_chunk_fwd(pre)
    assert rel_l2_slices(S_dec[n:n + 1], S_pre, axis_tokens=False)[0] < 1e-5
    assert np.linalg.norm(o_dec[n] - o_pre[-1]) / np.linalg.norm(o_pre[-1]) < 1e-5
