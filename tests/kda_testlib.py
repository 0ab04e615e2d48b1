"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
CPU oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import numpy as np

import kda_gen
import oracle

# Tolerances (max relative L2 error per (document, head) slice, O and final state):
# bf16-MFMA arithmetic 1e-2; fp32 verification arithmetic 1e-4.
TOL_BF16 = 1e-2
TOL_F32 = 1e-4
# Storing an output in bf16 (round to nearest even) alone contributes a relative
# error of at most 2^-8 per element, so an fp32-arithmetic run on bf16 inputs is
# held to 1e-4 on the fp32 states and to 2^-8 + 1e-4 on its bf16 outputs.
TOL_BF16_STORAGE = 2.0 ** -8


def rel_l2_slices(x, ref, cu=None, axis_tokens=True):
    """Max and global relative L2 error.  For outputs [T, H, D] the slices are
    (document, head); for states [N, H, D, D] they are (document, head)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    if axis_tokens:
        T, H = ref.shape[:2]
        bounds = [(0, T)] if cu is None else list(zip(cu[:-1], cu[1:]))
        for s, e in bounds:
            if e <= s:
                continue
            for h in range(H):
                den = np.linalg.norm(ref[s:e, h])
                if den > 0:
                    worst = max(worst, np.linalg.norm(x[s:e, h] - ref[s:e, h]) / den)
    else:
        N, H = ref.shape[:2]
        for n in range(N):
            for h in range(H):
                den = np.linalg.norm(ref[n, h])
                if den > 0:
                    worst = max(worst, np.linalg.norm(x[n, h] - ref[n, h]) / den)
    glob = np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300)
    return worst, glob


# Per-token bound on outputs: for every (document, head) slice and every token t
# of it, ||o_t - o_ref_t||_2 / max(||o_ref_t||_2, rms_t'(||o_ref_t'||_2)), the
# token's error against the larger of its own norm and the slice's
# root-mean-square token norm (the floor keeps near-zero outputs from dividing
# by almost nothing).  The slice tolerance above bounds an average of these;
# this bounds the worst single token, so one wrong token or a bad partial chunk
# cannot hide in a long slice.  bf16-MFMA arithmetic: 5e-2 (five times the
# slice tolerance); fp32 arithmetic: 1e-3, plus 2^-8 when O is stored in bf16
# (rounding a vector to bf16 moves it by at most 2^-8 of its own norm).
TOK_BF16 = 5e-2
TOK_F32 = 1e-3


def token_err_max(x, ref, cu=None, head_block=8):
    """Max over (document, head, token) of ||x_t - ref_t|| / max(||ref_t||, rms of
    ||ref_t'|| over the document's tokens of that head); outputs [T, H, D].
    Documents whose reference is all zero are skipped."""
    T, H = ref.shape[:2]
    bounds = [(0, T)] if cu is None else [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])]
    worst = 0.0
    for h0 in range(0, H, head_block):
        xs = np.asarray(x[:, h0:h0 + head_block], dtype=np.float64)
        rs = np.asarray(ref[:, h0:h0 + head_block], dtype=np.float64)
        en = np.sqrt(np.sum((xs - rs) ** 2, axis=-1))     # [T, hb]
        rn2 = np.sum(rs * rs, axis=-1)                      # [T, hb]
        for a, b in bounds:
            if b <= a:
                continue
            rms = np.sqrt(np.mean(rn2[a:b], axis=0))        # [hb]
            ok = rms > 0
            if np.any(ok):
                den = np.maximum(np.sqrt(rn2[a:b][:, ok]), rms[ok])
                worst = max(worst, float(np.max(en[a:b][:, ok] / den)))
    return worst


def _slice_f32(t, hs):
    """fp32 values of heads hs of a kda_gen.Tensor [T, H, ...], converting only the slice."""
    x = t.data[:, hs]
    return x.astype(np.float32) if t.dtype == "f32" else kda_gen.bf16_bits_to_f32(x)


def oracle_forward(inp, heads=None, group=8):
    """Oracle on a PrefillInputs, optionally on a subset of heads, in head groups
    to bound the fp64 working set."""
    heads = list(range(inp.H)) if heads is None else list(heads)
    T = inp.T
    o = np.zeros((T, len(heads), 128))
    S = np.zeros((inp.N, len(heads), 128, 128))
    for g0 in range(0, len(heads), group):
        hs = heads[g0:g0 + group]
        gg = oracle.gate_of(inp, _slice_f32(inp.z, hs).astype(np.float64), hs)
        S0 = None if inp.S0 is None else inp.S0[:, hs].astype(np.float64)
        qq, kk, bb = oracle.operands(inp, _slice_f32(inp.q, hs), _slice_f32(inp.k, hs),
                                     _slice_f32(inp.beta, hs))
        oo, SS = oracle.recurrent(qq, kk, _slice_f32(inp.v, hs), gg, bb, S0, inp.cu_seqlens)
        o[:, g0:g0 + len(hs)] = oo
        S[:, g0:g0 + len(hs)] = SS
    return o, S


def gpu_inputs(inp, device="cuda"):
    import torch
    t = {name: kda_gen.to_torch(getattr(inp, name), device) for name in ("q", "k", "v", "z", "beta")}
    t["A_log"] = torch.from_numpy(inp.A_log).to(device)
    t["S0"] = None if inp.S0 is None else torch.from_numpy(inp.S0).to(device)
    t["cu"] = torch.from_numpy(inp.cu_seqlens).to(device) if inp.N > 1 else None
    t["cu_host"] = inp.cu_seqlens if inp.N > 1 else None
    return t


def gpu_chunk_fwd(inp, compute=0, t=None, fused=False):
    """kda_chunk_fwd on the GPU; fused=True runs the single-kernel path (no
    workspace), otherwise the binding's default (two kernels for bf16 inputs)."""
    import linear_attention_fwd_amd as kda
    import torch
    t = t or gpu_inputs(inp)
    o, S = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min,
                             t["S0"], t["cu"], t["cu_host"], compute=compute,
                             workspace=False if fused else None, raw_inputs=inp.raw,
                             unbounded_gate=inp.gate == "softplus")
    torch.cuda.synchronize()
    return kda_gen.from_torch(o), kda_gen.from_torch(S)


def gpu_chunk_fwd_unbounded(inp, t=None, fused=False):
    """kda_chunk_fwd_unbounded (softplus gate) on the GPU: the two-kernel path for
    bf16 inputs (fused=True: the fused kernel), the fp32 fused kernel for fp32."""
    import linear_attention_fwd_amd as kda
    import torch
    t = t or gpu_inputs(inp)
    o, S = kda.kda_chunk_fwd_unbounded(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"],
                                       t["S0"], t["cu"], t["cu_host"], raw_inputs=inp.raw,
                                       workspace=False if fused else None)
    torch.cuda.synchronize()
    return kda_gen.from_torch(o), kda_gen.from_torch(S)


def gpu_segment_scan(inp, n_segments=0, compute=0, t=None):
    import linear_attention_fwd_amd as kda
    import torch
    t = t or gpu_inputs(inp)
    o, S = kda.kda_segment_scan(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"],
                                inp.g_min, t["S0"], t["cu"], t["cu_host"],
                                n_segments=n_segments, compute=compute, raw_inputs=inp.raw,
                                unbounded_gate=inp.gate == "softplus")
    torch.cuda.synchronize()
    return kda_gen.from_torch(o), kda_gen.from_torch(S)


def decode_gpu_inputs(inp, device="cuda"):
    import torch
    t = {name: kda_gen.to_torch(getattr(inp, name), device)
         for name in ("cq", "ck", "cv", "cz", "cbeta", "nq", "nk", "nv", "nz", "nbeta")}
    if inp.W2 > 0:
        for name in ("wq", "wk", "wv", "wz", "wbeta"):
            t[name] = kda_gen.to_torch(getattr(inp, name), device)
    t["A_log"] = torch.from_numpy(inp.A_log).to(device)
    t["accepted"] = torch.from_numpy(inp.accepted).to(device)
    t["state"] = torch.from_numpy(inp.state).to(device)
    return t


def gpu_decode(inp, t=None, state_slots=None, err_flag=None):
    import linear_attention_fwd_amd as kda
    import torch
    t = t or decode_gpu_inputs(inp)
    o = kda.kda_decode_step(t["state"], t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"],
                            t["accepted"], t["nq"], t["nk"], t["nv"], t["nz"], t["nbeta"],
                            t["A_log"], inp.g_min, state_slots=state_slots, err_flag=err_flag,
                            raw_inputs=inp.raw, unbounded_gate=inp.gate == "softplus")
    torch.cuda.synchronize()
    return kda_gen.from_torch(o), kda_gen.from_torch(t["state"])


def gpu_decode_window(inp, t=None, state_slots=None, err_flag=None):
    """kda_decode_step_window on ``inp`` (W2 > 0): (o bonus, o window, state)."""
    import linear_attention_fwd_amd as kda
    import torch
    t = t or decode_gpu_inputs(inp)
    o, ow = kda.kda_decode_step_window(
        t["state"], t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"], t["accepted"], t["nq"],
        t["nk"], t["nv"], t["nz"], t["nbeta"], t["wq"], t["wk"], t["wv"], t["wz"], t["wbeta"],
        t["A_log"], inp.g_min, state_slots=state_slots, err_flag=err_flag, raw_inputs=inp.raw,
        unbounded_gate=inp.gate == "softplus")
    torch.cuda.synchronize()
    return kda_gen.from_torch(o), kda_gen.from_torch(ow), kda_gen.from_torch(t["state"])


def oracle_checkpoints(inp, interval):
    """{(d, j): state after the first j * interval tokens of document d [H, dk, dv]}
    for every j >= 1 with j * interval < the document's length: the oracle's final
    state over that prefix of the document."""
    g_all = oracle.gate_of(inp, inp.z.f64())
    q_all, k_all, b_all = oracle.operands(inp, inp.q.f64(), inp.k.f64(), inp.beta.f64())
    cu = inp.cu_seqlens
    out = {}
    for d in range(inp.N):
        a, b = int(cu[d]), int(cu[d + 1])
        S0 = None if inp.S0 is None else inp.S0[d:d + 1].astype(np.float64)
        j = 1
        while j * interval < b - a:
            e = a + j * interval
            _, S = oracle.recurrent(q_all[a:e], k_all[a:e], inp.v.f64()[a:e], g_all[a:e],
                                    b_all[a:e], S0)
            out[(d, j)] = S[0]
            j += 1
    return out
