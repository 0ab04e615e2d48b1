"""Build rules checked on the compiled gfx950 code of every translation unit
(host-side, no GPU needed): packed fp32 VALU instructions are switched off at
compile time and must not appear; every global write goes through vector
memory, so no store, atomic, write-back or discard through the scalar data
cache may appear either.

This file names those instructions, so it is not sent to GPU machines (the
GPU runs load none of it).
"""
import re

import pytest

from test_asm_hazards import HIPCC, SOURCES, asm  # noqa: F401  (module fixture)

import os

PACKED_F32 = re.compile(r"^v_pk_(add|mul|fma|mov)_f32\b")
SCALAR_WRITE = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|"
                          r"dcache_discard)")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32(asm, src):  # noqa: F811
    bad = [l for l in asm[src] if PACKED_F32.match(l)]
    assert not bad, bad[:5]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_scalar_cache_writes(asm, src):  # noqa: F811
    bad = [l for l in asm[src] if SCALAR_WRITE.match(l)]
    assert not bad, bad[:5]


def test_patterns_match_what_they_look_for():
    assert PACKED_F32.match("v_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]")
    assert not PACKED_F32.match("v_pk_fma_f16 v0, v1, v2, v3")
    assert SCALAR_WRITE.match("s_store_dword s0, s[2:3], 0x0")
    assert SCALAR_WRITE.match("s_atomic_add s0, s[2:3], 0x0")
    assert not SCALAR_WRITE.match("s_load_dwordx4 s[0:3], s[4:5], 0x0")
