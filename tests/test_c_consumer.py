"""The C ABI from a plain C11 program (tests/c_consumer/kda_c_consumer.c): no
Python or PyTorch in the process, device memory from the HIP runtime's C API,
results checked against the fp64 C oracle inside the program."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_consumer", "kda_c_consumer")


def test_c_consumer_compiles(tmp_path):
    """The program builds as strict C11 (warnings are errors) against the header."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_consumer_build",
                                                  os.path.join(HERE, "c_consumer", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = os.path.join(os.path.dirname(HERE), "linear_attention_fwd_amd", "libkda.so")
    if not os.path.exists(lib):
        pytest.skip("libkda.so not built")
    out = str(tmp_path / "kda_c_consumer")
    r = subprocess.run(mod.command(out), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    assert os.path.exists(out)


@pytest.mark.gpu
def test_c_consumer_on_gpu():
    """fp32 prefill, bf16 two-kernel prefill with a caller workspace, and an fp32
    decode replay, each within tolerance of the oracle."""
    assert os.path.exists(BIN), "kda_c_consumer not built (run __graft_entry__.build())"
    print("[case] C consumer: fp32 prefill, bf16 prefill, fp32 decode", flush=True)
    r = subprocess.run([BIN], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    assert "all checks ok" in r.stdout
