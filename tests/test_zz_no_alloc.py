"""kda_chunk_fwd_noalloc (the prefill whose workspace is the library's static
device scratch) through the C ABI against kda_chunk_fwd with a caller
workspace: two calls in a row, the second with a smaller input, each equal to
kda_chunk_fwd bit for bit (same kernels on the same inputs) and within the
bf16 tolerance of the oracle."""
import numpy as np
import pytest

import kda_gen
from kda_testlib import TOL_BF16, gpu_inputs, oracle_forward, rel_l2_slices

pytestmark = pytest.mark.gpu


def _run(inp):
    import torch
    import linear_attention_fwd_amd as kda
    t = gpu_inputs(inp)
    o1, S1 = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min,
                               t["S0"], t["cu"], t["cu_host"])
    o2 = torch.full_like(o1, 7.0)
    S2 = torch.full_like(S1, 7.0)
    kda.kda_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A_log"], inp.g_min,
                              t["S0"], t["cu"], t["cu_host"], o=o2, final_state=S2)
    torch.cuda.synchronize()
    return (kda_gen.from_torch(o1), kda_gen.from_torch(S1), kda_gen.from_torch(o2),
            kda_gen.from_torch(S2))


def test_noalloc_equals_chunk_fwd_twice_smaller_second():
    import linear_attention_fwd_amd as kda
    big = kda_gen.make_prefill(61, 4000, 16, "bf16", lengths=[1500, 37, 0, 2463], s0_std=0.02,
                               s0_docs="all")
    small = kda_gen.make_prefill(62, 300, 4, "bf16", lengths=[130, 170])
    for inp in (big, small):
        need = kda.kda_chunk_fwd_workspace_size(inp.N, inp.T, inp.H)
        print(f"[case] noalloc T={inp.T} H={inp.H} N={inp.N} scratch {need} of "
              f"{kda.KDA_NOALLOC_SCRATCH_BYTES} bytes", flush=True)
        assert need <= kda.KDA_NOALLOC_SCRATCH_BYTES
        o1, S1, o2, S2 = _run(inp)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
        o_ref, S_ref = oracle_forward(inp)
        eo, _ = rel_l2_slices(o2, o_ref, inp.cu_seqlens)
        es, _ = rel_l2_slices(S2, S_ref, axis_tokens=False)
        print(f"    O {eo:.3e}  S {es:.3e}", flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_refuses_sizes_beyond_its_scratch():
    import torch
    import linear_attention_fwd_amd as kda
    T, H = 8192, 96
    assert kda.kda_chunk_fwd_workspace_size(1, T, H) > kda.KDA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_fwd_noalloc(x, x, x, x, b)
    assert e.value.code == -6
