"""Host-side check of the generated gfx950 code (no GPU needed).

The global -> LDS copies of the recurrence kernel are issued through inline
asm, which the compiler's hazard recognizer does not look into.  The hardware
needs 5 wait states between a VALU write of an SGPR (v_readfirstlane builds
the buffer descriptor) and a vector memory read of it, and 1 between an SALU
write of M0 and an LDS-DMA load; without them the load can use a stale
descriptor.  Every LDS-DMA load in the compiled kernels must therefore be
directly preceded by s_nop 4.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["kda_split.hip"])
def test_lds_dma_loads_have_wait_states(tmp_path, src):
    out = tmp_path / "k.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops", "-I",
                    os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    lines = [l.strip() for l in out.read_text().splitlines()
             if l.strip() and not l.strip().startswith(";")]
    dma = [i for i, l in enumerate(lines) if l.startswith("buffer_load") and l.endswith(" lds")]
    assert dma, "expected global -> LDS loads in the recurrence kernel"
    unguarded = [lines[i] for i in dma if lines[i - 1] != "s_nop 4"]
    assert not unguarded, unguarded
