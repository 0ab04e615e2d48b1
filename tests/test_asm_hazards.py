"""Host-side check of the generated gfx950 code (no GPU needed).

The global -> LDS copies of the recurrence kernel are issued through inline
asm (helpers in kda_device.h, which every translation unit includes), and the
compiler's hazard recognizer does not look into inline asm.  The hardware
needs 5 wait states between a VALU write of an SGPR (v_readfirstlane builds
the buffer descriptor) and a vector memory read of it, and 1 between an SALU
write of M0 and an LDS-DMA load; without them the load can use a stale
descriptor.  Every LDS-DMA load in every compiled translation unit must
therefore be directly preceded by s_nop 4.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "*.hip")))


def device_asm(src, out_dir):
    """gfx950 assembly of one translation unit, built with the library's flags;
    comment lines dropped."""
    out = os.path.join(out_dir, src + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops", "-I",
                    os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    os.path.join(CSRC, src), "-o", out],
                   check=True, capture_output=True)
    with open(out, encoding="utf-8") as fh:
        return [l.strip() for l in fh if l.strip() and not l.strip().startswith(";")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    return {src: device_asm(src, d) for src in SOURCES}


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_lds_dma_loads_have_wait_states(asm, src):
    lines = asm[src]
    dma = [i for i, l in enumerate(lines) if l.startswith("buffer_load") and l.endswith(" lds")]
    unguarded = [lines[i] for i in dma if lines[i - 1] != "s_nop 4"]
    assert not unguarded, unguarded


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_recurrence_uses_lds_dma(asm):
    lines = asm["kda_split.hip"]
    assert any(l.startswith("buffer_load") and l.endswith(" lds") for l in lines), \
        "expected global -> LDS loads in the recurrence kernel"
