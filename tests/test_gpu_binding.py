"""The Python binding refuses caller-supplied outputs and workspaces it cannot
hand to the library safely: the C interface takes bare pointers, so an output
of the wrong shape, dtype or device would be written out of bounds.  Every case
raises before anything is launched."""
import pytest

import kda_gen
from kda_testlib import decode_gpu_inputs, gpu_inputs

pytestmark = pytest.mark.gpu


def _prefill():
    inp = kda_gen.make_prefill(91, 130, 2, "bf16")
    return inp, gpu_inputs(inp)


def _args(t, inp):
    return (t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min, None, None, None)


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_segment_scan",
                                "kda_chunk_fwd_checkpoints", "kda_chunk_fwd_unbounded"])
def test_prefill_outputs_checked(fn):
    import torch
    import linear_attention_fwd_amd as kda
    inp, t = _prefill()
    print(f"[case] binding checks, {fn}", flush=True)
    T, H = inp.T, inp.H
    f = getattr(kda, fn)

    def call(**kw):
        if fn == "kda_chunk_fwd_checkpoints":
            return f(t["q"], t["k"], t["v"], t["z"], t["beta"], 64, t["A_log"], inp.g_min, **kw)
        if fn == "kda_chunk_fwd_unbounded":
            return f(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], **kw)
        return f(*_args(t, inp), **kw)

    bad_o = [torch.empty((T - 1, H, 128), dtype=torch.bfloat16, device="cuda"),     # short
             torch.empty((T, H, 128), dtype=torch.float32, device="cuda"),          # dtype
             torch.empty((T, H, 256), dtype=torch.bfloat16, device="cuda")[..., :128],  # strided
             torch.empty((T, H, 128), dtype=torch.bfloat16)]                        # host
    for o in bad_o:
        with pytest.raises((ValueError, TypeError)):
            call(o=o)
    for S in (torch.empty((1, H, 128, 127), dtype=torch.float32, device="cuda"),
              torch.empty((1, H, 128, 128), dtype=torch.bfloat16, device="cuda")):
        with pytest.raises((ValueError, TypeError)):
            call(final_state=S)
    if fn not in ("kda_chunk_fwd_noalloc",):
        with pytest.raises(ValueError):
            call(workspace=torch.empty(1 << 20, dtype=torch.uint8))  # host memory
    o, S = call()[:2]  # the same call with its own outputs runs
    torch.cuda.synchronize()
    assert o.shape == (T, H, 128) and S.shape == (1, H, 128, 128)


def test_recurrence_outputs_checked():
    import torch
    import linear_attention_fwd_amd as kda
    inp, t = _prefill()
    ws = torch.empty(kda.kda_chunk_fwd_workspace_size(1, inp.T, inp.H), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(ValueError):
        kda.kda_chunk_recurrence(t["v"], ws, o=torch.empty((inp.T, inp.H + 1, 128),
                                                           dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        kda.kda_chunk_prep(t["q"], t["k"], t["z"], t["beta"], torch.empty(16, dtype=torch.uint8))


def test_decode_outputs_checked():
    import torch
    import linear_attention_fwd_amd as kda
    inp = kda_gen.make_decode(92, 6, 2, 4, "bf16", W2=2)
    t = decode_gpu_inputs(inp)
    print("[case] binding checks, decode", flush=True)
    base = (t["state"], t["cq"], t["ck"], t["cv"], t["cz"], t["cbeta"], t["accepted"], t["nq"],
            t["nk"], t["nv"], t["nz"], t["nbeta"])
    with pytest.raises(ValueError):
        kda.kda_decode_step(*base, t["A_log"], inp.g_min,
                            o=torch.empty((5, 2, 128), dtype=torch.bfloat16, device="cuda"))
    win = (t["wq"], t["wk"], t["wv"], t["wz"], t["wbeta"])
    with pytest.raises(ValueError):
        kda.kda_decode_step_window(*base, *win, t["A_log"], inp.g_min,
                                   o_window=torch.empty((6, 1, 2, 128), dtype=torch.bfloat16,
                                                        device="cuda"))
