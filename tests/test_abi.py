"""Host-side checks of the C ABI (no GPU needed).

* libkda.so loads and exports every function include/kda.h declares;
* invalid arguments are rejected with the documented status before any HIP
  call (so nothing here touches a device: every call below fails validation).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import linear_attention_fwd_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE = 0, -1, -2, -3
KDA_ERR_GATE_BOUND, KDA_ERR_SEQLENS, KDA_ERR_WORKSPACE = -4, -5, -6
KDA_ERR_UNSUPPORTED = -8


def declared_functions():
    with open(HEADER, encoding="utf-8") as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kda_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from linear_attention_fwd_amd import _build
        _build.build()
    return kda.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kda_chunk_fwd", "kda_segment_scan", "kda_decode_step"):
        assert required in names
    assert set(names) == set(kda.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(kda_[a-z_0-9]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(-4) == b"KDA_ERR_GATE_BOUND"
    assert lib.kda_status_string(12345) == b"KDA_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _prefill(lib, fn="kda_chunk_fwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A=None, g_min=-5.0, S0=None, cu=None,
             cu_host=None, N=1, T=128, H=4, dk=128, dv=128, dtype=1, compute=0, o=FAKE,
             fin=FAKE, nseg=0, ws=None, ws_bytes=0)
    a.update(kw)
    args = [a["q"], a["k"], a["v"], a["g"], a["beta"], a["A"], a["g_min"], a["S0"], a["cu"],
            a["cu_host"], a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"], a["compute"]]
    if fn == "kda_chunk_fwd":
        return lib.kda_chunk_fwd(*args, a["o"], a["fin"], a["ws"], a["ws_bytes"], None)
    return lib.kda_segment_scan(*args, a["nseg"], a["o"], a["fin"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_segment_scan"])
def test_prefill_validation(lib, fn):
    assert _prefill(lib, fn, q=None) == KDA_ERR_NULL
    assert _prefill(lib, fn, o=None) == KDA_ERR_NULL
    assert _prefill(lib, fn, dk=64) == KDA_ERR_SHAPE
    assert _prefill(lib, fn, dv=256) == KDA_ERR_SHAPE
    assert _prefill(lib, fn, H=0) == KDA_ERR_SHAPE
    assert _prefill(lib, fn, T=-1) == KDA_ERR_SHAPE
    assert _prefill(lib, fn, dtype=7) == KDA_ERR_DTYPE
    assert _prefill(lib, fn, compute=3) == KDA_ERR_DTYPE
    # the subtile factors need 16 * |g_min| < 88: g_min below -5 is refused
    assert _prefill(lib, fn, g_min=-5.5) == KDA_ERR_GATE_BOUND
    assert _prefill(lib, fn, g_min=0.0) == KDA_ERR_GATE_BOUND
    assert _prefill(lib, fn, g_min=float("nan")) == KDA_ERR_GATE_BOUND
    # N > 1 needs offsets; offsets need a host copy, start at 0, increase, end at T
    assert _prefill(lib, fn, N=2) == KDA_ERR_SEQLENS
    good = (ctypes.c_int32 * 3)(0, 50, 128)
    assert _prefill(lib, fn, N=2, cu=FAKE) == KDA_ERR_SEQLENS
    for bad in ((1, 50, 128), (0, 90, 60), (0, 50, 127)):
        arr = (ctypes.c_int32 * 3)(*bad)
        assert _prefill(lib, fn, N=2, cu=FAKE, cu_host=ctypes.cast(arr, ctypes.c_void_p)) \
            == KDA_ERR_SEQLENS
    assert good[2] == 128


def test_segment_scan_workspace_checks(lib):
    # explicit segment count: a short or missing workspace is refused before any launch
    # enough for either path: chunk images + pairs of the chunk-slot segments +
    # pairs and entry states of their groups (bf16), or pairs + entry states of
    # the token segments (fp32)
    need = lib.kda_segment_scan_workspace_size(1, 128, 4, 4, 128, 128)
    slots = 128 // 64 + 1                                    # 3 chunk slots -> 3 segments
    # images + segment pairs, and pairs + entry states of the 2 groups of 2 segments
    # the pairs are scanned in
    need_bf16 = slots * 4 * 62464 + 256 + 3 * 4 * 128 * 256 * 4 + 2 * 4 * 128 * 384 * 4
    need_f32 = 4 * 4 * 128 * 384 * 4                         # 4 token segments
    assert need == max(need_bf16, need_f32)
    assert lib.kda_segment_scan_workspace_size(0, 128, 4, 4, 128, 128) == 0
    assert lib.kda_segment_scan_workspace_size(1, 128, 4, 4, 64, 128) == 0
    for compute, req in ((0, need_bf16), (1, need_f32)):  # bf16 inputs, both arithmetic paths
        assert _prefill(lib, "kda_segment_scan", nseg=4, compute=compute, ws=None,
                        ws_bytes=0) == KDA_ERR_WORKSPACE
        assert _prefill(lib, "kda_segment_scan", nseg=4, compute=compute, ws=FAKE,
                        ws_bytes=req - 1) == KDA_ERR_WORKSPACE
        assert _prefill(lib, "kda_segment_scan", nseg=4, compute=compute,
                        ws=ctypes.c_void_p(0x1004), ws_bytes=req) == KDA_ERR_WORKSPACE
    assert _prefill(lib, "kda_segment_scan", nseg=4, S0=FAKE, fin=FAKE, ws=FAKE,
                    ws_bytes=need) == KDA_ERR_UNSUPPORTED


def test_chunk_fwd_workspace_checks(lib):
    # one 61 KiB chunk image per head and slot, floor(T / 64) + N slots per head,
    # then the document order (4 bytes per document, rounded up to 256)
    need = lib.kda_chunk_fwd_workspace_size(1, 128, 4, 128, 128)
    assert need == (128 // 64 + 1) * 4 * 62464 + 256
    assert lib.kda_chunk_fwd_workspace_size(3, 1000, 2, 128, 128) == \
        (1000 // 64 + 3) * 2 * 62464 + 256
    assert lib.kda_chunk_fwd_workspace_size(65, 1000, 2, 128, 128) == \
        (1000 // 64 + 65) * 2 * 62464 + 512
    assert lib.kda_chunk_fwd_workspace_size(0, 128, 4, 128, 128) == 0
    assert lib.kda_chunk_fwd_workspace_size(1, 128, 4, 64, 128) == 0
    # the two-kernel path (bf16, compute AUTO) refuses a short or misaligned workspace
    assert _prefill(lib, ws=FAKE, ws_bytes=need - 1) == KDA_ERR_WORKSPACE
    assert _prefill(lib, ws=ctypes.c_void_p(0x1004), ws_bytes=need) == KDA_ERR_WORKSPACE


def test_prep_and_recurrence_validation(lib):
    need = lib.kda_chunk_fwd_workspace_size(1, 128, 4, 128, 128)

    def prep(**kw):
        a = dict(q=FAKE, g_min=-5.0, N=1, T=128, H=4, dk=128, dtype=1, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return lib.kda_chunk_prep(a["q"], FAKE, FAKE, FAKE, None, a["g_min"], None, None, a["N"],
                                  a["T"], a["H"], a["dk"], 128, a["dtype"], a["ws"], a["ws_bytes"],
                                  None)

    def rec(**kw):
        a = dict(v=FAKE, o=FAKE, N=1, T=128, H=4, dtype=1, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return lib.kda_chunk_recurrence(a["v"], None, None, None, a["N"], a["T"], a["H"], 128, 128,
                                        a["dtype"], a["ws"], a["ws_bytes"], a["o"], None, None)

    assert prep(q=None) == KDA_ERR_NULL
    assert prep(dk=64) == KDA_ERR_SHAPE
    assert prep(g_min=-6.0) == KDA_ERR_GATE_BOUND
    assert prep(dtype=0) == KDA_ERR_UNSUPPORTED      # bf16 inputs only
    assert prep(ws=None) == KDA_ERR_WORKSPACE
    assert prep(ws_bytes=need - 1) == KDA_ERR_WORKSPACE
    assert prep(N=2) == KDA_ERR_SEQLENS
    assert prep(T=0) == KDA_OK                       # nothing to do, nothing launched
    assert rec(v=None) == KDA_ERR_NULL
    assert rec(o=None) == KDA_ERR_NULL
    assert rec(H=0) == KDA_ERR_SHAPE
    assert rec(dtype=0) == KDA_ERR_UNSUPPORTED
    assert rec(ws=ctypes.c_void_p(0x1008)) == KDA_ERR_WORKSPACE
    assert rec(ws_bytes=0) == KDA_ERR_WORKSPACE


def test_checkpoint_validation(lib):
    # one entry per interval / 64 chunk slots: (floor(T / 64) + N - 1) // (interval / 64) + 1
    assert lib.kda_checkpoint_count(1, 8192, 512) == (8192 // 64 + 1 - 1) // 8 + 1
    assert lib.kda_checkpoint_count(3, 1000, 128) == (1000 // 64 + 3 - 1) // 2 + 1
    assert lib.kda_checkpoint_count(1, 1000, 100) == 0      # not a multiple of 64
    assert lib.kda_checkpoint_count(0, 1000, 128) == 0
    ws = lib.kda_chunk_fwd_workspace_size(1, 128, 4, 128, 128)
    nck = lib.kda_checkpoint_count(1, 128, 64) * 4 * 128 * 128 * 4

    def call(**kw):
        a = dict(q=FAKE, g_min=-5.0, N=1, T=128, H=4, dk=128, dtype=1, interval=64, ck=FAKE,
                 ck_bytes=nck, o=FAKE, ws=FAKE, ws_bytes=ws)
        a.update(kw)
        return lib.kda_chunk_fwd_checkpoints(a["q"], FAKE, FAKE, FAKE, FAKE, None, a["g_min"], None,
                                             None, None, a["N"], a["T"], a["H"], a["dk"], 128,
                                             a["dtype"], a["interval"], a["ck"], a["ck_bytes"],
                                             a["o"], None, a["ws"], a["ws_bytes"], None)
    assert call(q=None) == KDA_ERR_NULL
    assert call(dk=64) == KDA_ERR_SHAPE
    assert call(dtype=0) == KDA_ERR_UNSUPPORTED          # bf16 two-kernel path only
    assert call(interval=0) == KDA_ERR_SHAPE
    assert call(interval=96) == KDA_ERR_SHAPE
    assert call(ck=None) == KDA_ERR_NULL
    assert call(ck_bytes=nck - 1) == KDA_ERR_WORKSPACE
    assert call(ws=None) == KDA_ERR_WORKSPACE
    assert call(ws_bytes=ws - 1) == KDA_ERR_WORKSPACE
    assert call(g_min=-6.0) == KDA_ERR_GATE_BOUND


def test_decode_validation(lib):
    def call(**kw):
        a = dict(state=FAKE, pool=8, slots=None, c=FAKE, acc=FAKE, W=4, n=FAKE, A=None,
                 g_min=-5.0, o=FAKE, err=None, N=8, H=4, dk=128, dv=128, dtype=1)
        a.update(kw)
        c, n = a["c"], a["n"]
        return lib.kda_decode_step(a["state"], a["pool"], a["slots"], c, c, c, c, c, a["acc"],
                                   a["W"], n, n, n, n, n, a["A"], a["g_min"], a["o"], a["err"],
                                   a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)
    assert call(state=None) == KDA_ERR_NULL
    # the pool: without slots every sequence needs its own state; with slots the
    # kernel skips any slot outside [0, S_pool) (checked there, not here)
    assert call(pool=7) == KDA_ERR_SHAPE
    assert call(pool=-1) == KDA_ERR_SHAPE
    assert call(pool=-1, slots=FAKE) == KDA_ERR_SHAPE
    assert call(pool=1, slots=FAKE, state=None) == KDA_ERR_NULL  # a small pool is fine with slots
    assert call(pool=(1 << 31) - 1, H=4, state=None) == KDA_ERR_SHAPE  # S_pool * H overflows
    assert call(H=65536) == KDA_ERR_SHAPE
    assert call(acc=None) == KDA_ERR_NULL
    assert call(n=None) == KDA_ERR_NULL
    assert call(c=None) == KDA_ERR_NULL          # drafts needed when W > 0
    assert call(dk=64) == KDA_ERR_SHAPE
    assert call(W=-1) == KDA_ERR_SHAPE
    assert call(H=0) == KDA_ERR_SHAPE
    assert call(dtype=5) == KDA_ERR_DTYPE
    assert call(g_min=-6.0) == KDA_ERR_GATE_BOUND
    assert call(N=0) == KDA_OK                   # nothing to do, nothing launched
    assert lib.kda_last_error() is not None


def test_raw_inputs_flag(lib):
    """KDA_RAW_INPUTS is refused only where the normalised rows would lose
    precision (bf16 inputs into fp32 arithmetic); other bits are unknown.  (The accepted combinations would launch kernels, so
    they are driven here only by the sanitizer build against stub launchers.)"""
    RAW = kda.KDA_RAW_INPUTS
    def fwd(dtype, ws, compute=0):
        return lib.kda_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, None, 1,
                                 256, 4, 128, 128, dtype, compute, FAKE, None, ws,
                                 1 << 30 if ws else 0, None)
    assert fwd(1 | RAW, FAKE, compute=1) == KDA_ERR_UNSUPPORTED  # bf16 in, fp32 arithmetic
    assert fwd(1 | RAW, None, compute=1) == KDA_ERR_UNSUPPORTED
    assert fwd(1 | 0x400, FAKE) == KDA_ERR_DTYPE              # unknown bit
    for n_seg in (0, 7):  # refused before the device is asked for its compute units
        # (bf16 inputs, fp32 arithmetic)
        assert lib.kda_segment_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, None, 1,
                                    256, 4, 128, 128, 1 | RAW, 1, n_seg, FAKE, None, FAKE, 1 << 30,
                                    None) == KDA_ERR_UNSUPPORTED
    # accepted by decode (rejected here only for the missing state)
    assert lib.kda_decode_step(None, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE,
                               FAKE, FAKE, FAKE, None, -5.0, FAKE, None, 8, 4, 128, 128, 1 | RAW,
                               None) == KDA_ERR_NULL


def test_unbounded_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, T=256, H=4, dtype=1, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        q = a["q"]
        return lib.kda_chunk_fwd_unbounded(q, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 1,
                                           a["T"], a["H"], 128, 128, a["dtype"], FAKE, None,
                                           a["ws"], a["ws_bytes"], None)
    assert call(q=None) == KDA_ERR_NULL
    assert call(ws_bytes=100) == KDA_ERR_WORKSPACE  # a workspace given must be large enough
    assert call(dtype=0, H=0) == KDA_ERR_SHAPE      # fp32 inputs (fused kernel) validated too
    assert call(dtype=0, q=None) == KDA_ERR_NULL
    assert call(H=0) == KDA_ERR_SHAPE


def test_decode_window_validation(lib):
    def call(**kw):
        a = dict(state=FAKE, pool=8, c=FAKE, acc=FAKE, W=4, n=FAKE, w=FAKE, W2=4, o=FAKE, ow=FAKE,
                 N=8, H=4, dtype=1)
        a.update(kw)
        c, n, w = a["c"], a["n"], a["w"]
        return lib.kda_decode_step_window(a["state"], a["pool"], None, c, c, c, c, c, a["acc"],
                                          a["W"], n, n,
                                          n, n, n, w, w, w, w, w, a["W2"], None, -5.0, a["o"],
                                          a["ow"], None, a["N"], a["H"], 128, 128, a["dtype"],
                                          None)
    assert call(w=None) == KDA_ERR_NULL          # window inputs needed when W2 > 0
    assert call(ow=None) == KDA_ERR_NULL
    assert call(W2=-1) == KDA_ERR_SHAPE
    assert call(dtype=5) == KDA_ERR_DTYPE
    assert call(state=None) == KDA_ERR_NULL
    assert call(pool=4) == KDA_ERR_SHAPE
    assert call(N=0) == KDA_OK


def test_segment_scan_refuses_overlapping_states(lib):
    """kda_segment_scan runs the segments of a document concurrently, so its
    final states must not overlap the initial states: exact aliasing and partial
    overlaps in either direction are refused before anything is launched, and
    adjacent ranges are accepted (then refused for the missing workspace)."""
    N, H = 3, 4
    nbytes = N * H * 128 * 128 * 4
    base = 1 << 32

    def call(init, fin, ws=None):
        return lib.kda_segment_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, ctypes.c_void_p(init),
                                    FAKE, np.array([0, 64, 128, 256], np.int32).ctypes.data_as(
                                        ctypes.c_void_p), N, 256, H, 128, 128, 1, 0, 7, FAKE,
                                    ctypes.c_void_p(fin), ws, 0, None)
    assert call(base, base) == KDA_ERR_UNSUPPORTED
    assert call(base, base + 4096) == KDA_ERR_UNSUPPORTED
    assert call(base + nbytes - 4, base) == KDA_ERR_UNSUPPORTED
    assert call(base, base + nbytes - 4) == KDA_ERR_UNSUPPORTED
    assert call(base, base + nbytes) == KDA_ERR_WORKSPACE     # adjacent: no overlap
    assert call(base + nbytes, base) == KDA_ERR_WORKSPACE


def test_head_count_bound(lib):
    """H above 65535 would overflow the kernels' 32-bit chunk offsets (64 tokens
    x H x 128 channels x 4 bytes): refused by every prefill entry point."""
    big = 65536
    ok = 65535
    assert lib.kda_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, None, 1, 256,
                             big, 128, 128, 1, 0, FAKE, None, None, 0, None) == KDA_ERR_SHAPE
    assert lib.kda_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, None, 1, 256,
                             ok, 128, 128, 1, 0, FAKE, None, FAKE, 0, None) == KDA_ERR_WORKSPACE
    assert lib.kda_chunk_prep(FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, 1, 256, big, 128,
                              128, 1, FAKE, 1 << 40, None) == KDA_ERR_SHAPE
    assert lib.kda_segment_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, -5.0, None, None, None, 1, 256,
                                big, 128, 128, 1, 0, 7, FAKE, None, FAKE, 1 << 40,
                                None) == KDA_ERR_SHAPE
    assert lib.kda_chunk_fwd_unbounded(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 1, 256,
                                       big, 128, 128, 1, FAKE, None, FAKE, 1 << 40,
                                       None) == KDA_ERR_SHAPE


def test_launch_size_bounds(lib):
    """Sizes whose kernels would exceed one dispatch (2^32 - 1 work-items) are
    refused before anything is enqueued; the largest accepted sizes pass the
    shape checks (and then fail on the missing workspace or state instead)."""
    H = 65535
    WS = -6  # KDA_ERR_WORKSPACE

    def docs(n):  # n documents of 64 tokens
        cu = (ctypes.c_int32 * (n + 1))(*range(0, 64 * (n + 1), 64))
        return dict(N=n, T=64 * n, H=H, cu=FAKE, cu_host=ctypes.cast(cu, ctypes.c_void_p)), cu

    kw, keep = docs(128)   # N * H = 8 388 480, slots * H = 16 776 960
    assert _prefill(lib, "kda_chunk_fwd", ws=FAKE, **kw) == WS
    kw, keep = docs(129)   # N * H = 8 454 015
    assert _prefill(lib, "kda_chunk_fwd", ws=FAKE, **kw) == KDA_ERR_SHAPE
    assert _prefill(lib, "kda_segment_scan", nseg=4, **kw) == KDA_ERR_SHAPE
    # chunk slots x heads: floor(T / 64) + N slots
    assert _prefill(lib, "kda_chunk_fwd", T=64 * 255, H=H, ws=FAKE) == WS           # 256 slots
    assert _prefill(lib, "kda_chunk_fwd", T=64 * 256, H=H, ws=FAKE) == KDA_ERR_SHAPE  # 257
    # segment scan: segments x heads <= 4 194 296 (64 segments at H = 65535)
    for compute in (0, 1):
        assert _prefill(lib, "kda_segment_scan", T=64 * 65, H=H, nseg=64,
                        compute=compute) == WS
        assert _prefill(lib, "kda_segment_scan", T=64 * 65, H=H, nseg=65,
                        compute=compute) == KDA_ERR_SHAPE

    def dec(N, state):
        return lib.kda_decode_step(state, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, None, -5.0, FAKE, None, N, H, 128, 128,
                                   1, None)
    assert dec(256, None) == KDA_ERR_NULL    # N * H = 16 776 960: shape accepted
    assert dec(257, FAKE) == KDA_ERR_SHAPE   # 16 842 495


def test_one_hip_runtime_per_process():
    """Loading the library before torch has touched anything must not bring in a
    second HIP runtime (PyTorch ships its own; with two in one process the one
    initialised second sees no GPU)."""
    code = ("import os, linear_attention_fwd_amd as kda\n"
            "kda.load_library()\n"
            "import torch\n"
            "maps = open(f'/proc/{os.getpid()}/maps').read()\n"
            "print(len(set(l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l)))\n")
    out = subprocess.run([__import__("sys").executable, "-c", code], capture_output=True,
                         text=True, cwd=ROOT, check=True).stdout
    assert out.strip() == "1", out


@pytest.mark.parametrize("lang,std", [("c", "c99"), ("c++", "c++11")])
def test_header_is_plain_c(lang, std, tmp_path):
    """include/kda.h compiles on its own as C99 and C++11 with warnings as
    errors, and a C caller can take the address of every declared function."""
    compiler = "gcc" if lang == "c" else "g++"
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    funcs = declared_functions()
    body = "\n".join(f"  p = (const void *)&{f}; (void)p;" for f in funcs)
    src.write_text(f'#include "kda.h"\nint main(void) {{\n  const void *p;\n{body}\n  return 0;\n}}\n')
    r = subprocess.run([compiler, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", f"-std={std}",
                        "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None)
@given(lengths=st.lists(st.integers(0, 3000), min_size=1, max_size=20),
       interval=st.sampled_from([64, 128, 192, 512, 1024]))
def test_checkpoint_indices_are_unique_and_in_range(lib, lengths, interval):
    """Every checkpoint the header documents, index
    (floor(cu[d] / 64) + d + j * interval / 64 - 1) / (interval / 64) for
    j * interval < length of d, lies below kda_checkpoint_count and no two
    (document, j) share one."""
    N, T = len(lengths), sum(lengths)
    count = lib.kda_checkpoint_count(N, T, interval)
    assert count >= 1
    cu = np.concatenate([[0], np.cumsum(lengths)])
    step = interval // 64
    seen = set()
    for d, L in enumerate(lengths):
        j = 1
        while j * interval < L:
            idx = (cu[d] // 64 + d + j * step - 1) // step
            assert 0 <= idx < count
            assert idx not in seen
            seen.add(idx)
            j += 1


@settings(max_examples=60, deadline=None)
@given(N=st.integers(1, 5000), T=st.integers(0, 1 << 24), H=st.integers(1, 128))
def test_workspace_size_formula(lib, N, T, H):
    """One 61 KiB image per head and chunk slot (floor(T / 64) + N slots), then
    4 bytes per document rounded up to 256; no 32-bit overflow."""
    want = (T // 64 + N) * H * 62464 + (4 * N + 255) // 256 * 256
    assert lib.kda_chunk_fwd_workspace_size(N, T, H, 128, 128) == want


def test_unbounded_gate_flag(lib):
    """KDA_UNBOUNDED_GATE: the entry points neither use nor check g_min under the
    unbounded gate (-7 would be refused by the bounded one).  (The accepted calls
    would launch kernels; they stop here at a later check: the workspace, or the
    missing decode state.)"""
    G = kda.KDA_UNBOUNDED_GATE
    assert _prefill(lib, "kda_chunk_fwd", g_min=-7.0, ws=FAKE) == KDA_ERR_GATE_BOUND
    assert _prefill(lib, "kda_chunk_fwd", g_min=-7.0, ws=FAKE, dtype=1 | G) == KDA_ERR_WORKSPACE
    assert _prefill(lib, "kda_segment_scan", g_min=-7.0, nseg=4) == KDA_ERR_GATE_BOUND
    assert _prefill(lib, "kda_segment_scan", g_min=-7.0, nseg=4, dtype=1 | G) == KDA_ERR_WORKSPACE
    def dec(dtype, state):
        return lib.kda_decode_step(state, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, None, -7.0, FAKE, None, 8, 4, 128, 128,
                                   dtype, None)
    assert dec(1, FAKE) == KDA_ERR_GATE_BOUND
    assert dec(1 | G, None) == KDA_ERR_NULL
