"""Python binding of libkda.so, the MI355X (gfx950) Kimi Delta Attention forward.

Argument marshalling only: every step of the operator runs in the HIP kernels
behind the C ABI declared in ``include/kda.h``.  PyTorch provides device memory
and the current stream.  There is no fallback: if the library is missing or the
tensors are not on a GPU, calls raise.

Every compute function takes ``raw_inputs=True`` for q, k not yet L2-normalised
and beta given as a logit (the kernels then normalise and apply the sigmoid;
KDA_RAW_INPUTS in the C ABI).

Entry points (same names as the C ABI):
  * ``kda_chunk_fwd``    -- chunkwise prefill of packed documents
  * ``kda_chunk_fwd_noalloc`` -- the same with the library's static device scratch
  * ``kda_chunk_fwd_unbounded`` -- the same with the unbounded (softplus) gate
  * ``kda_segment_scan`` -- prefill with intra-device segment pairs + scan
  * ``kda_decode_step``  -- decode step with speculative-verify replay
  * ``kda_decode_step_window`` -- the same step fused with the next draft window
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_RAW_INPUTS = 0x100  # OR'ed into dtype: q, k unnormalised and beta a logit
KDA_UNBOUNDED_GATE = 0x200  # OR'ed into dtype: g = -exp(A) softplus(z) instead of the bounded gate
KDA_COMPUTE_AUTO, KDA_COMPUTE_F32 = 0, 1
KDA_DECODE_ERR_ACCEPTED, KDA_DECODE_ERR_SLOT = 1, 2  # bits of a decode step's err_flag
STATUS = {0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_DTYPE",
          -4: "KDA_ERR_GATE_BOUND", -5: "KDA_ERR_SEQLENS", -6: "KDA_ERR_WORKSPACE",
          -7: "KDA_ERR_HIP", -8: "KDA_ERR_UNSUPPORTED"}
EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_unbounded",
           "kda_chunk_fwd_workspace_size",
           "kda_chunk_prep",
           "kda_chunk_recurrence", "kda_chunk_fwd_checkpoints", "kda_checkpoint_count",
           "kda_segment_scan",
           "kda_segment_scan_workspace_size",
           "kda_default_segments", "kda_decode_step", "kda_decode_step_window", "kda_status_string",
           "kda_last_error")

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__(f"{STATUS.get(code, code)}: {detail}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with linear_attention_fwd_amd._build.build()")
    # PyTorch ships its own HIP runtime.  Import it first so that libkda.so binds
    # to that runtime (same soname, already loaded) instead of loading a second
    # one from /opt/rocm: with two HIP runtimes in one process whichever
    # initialises second finds no GPU.
    _torch()
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    prefill = [vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd.argtypes = prefill + [vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = prefill[:-1] + [vp, vp, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_unbounded.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                            i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_fwd_unbounded.restype = ctypes.c_int
    lib.kda_chunk_fwd_checkpoints.argtypes = prefill[:-1] + [i32, vp, ctypes.c_size_t, vp, vp, vp,
                                                             ctypes.c_size_t, vp]
    lib.kda_chunk_fwd_checkpoints.restype = ctypes.c_int
    lib.kda_checkpoint_count.argtypes = [i32, i64, i32]
    lib.kda_checkpoint_count.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_prep.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, i32, i64, i32, i32, i32, i32,
                                   vp, ctypes.c_size_t, vp]
    lib.kda_chunk_prep.restype = ctypes.c_int
    lib.kda_chunk_recurrence.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp,
                                         ctypes.c_size_t, vp, vp, vp]
    lib.kda_chunk_recurrence.restype = ctypes.c_int
    lib.kda_segment_scan.argtypes = prefill + [i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_segment_scan.restype = ctypes.c_int
    lib.kda_segment_scan_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kda_segment_scan_workspace_size.restype = ctypes.c_size_t
    lib.kda_default_segments.argtypes = []
    lib.kda_default_segments.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                    vp, f32, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step_window.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, i32, vp, f32, vp, vp, vp, i32, i32,
                                           i32, i32, i32, vp]
    lib.kda_decode_step_window.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise KDAError(rc, _lib.kda_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t, raw_inputs: bool = False, unbounded_gate: bool = False) -> int:
    """dtype argument of the C ABI for tensor t, with KDA_RAW_INPUTS when q, k are
    unnormalised and beta is a logit (the kernels normalise and apply the sigmoid)
    and KDA_UNBOUNDED_GATE for the unbounded gate."""
    torch = _torch()
    flag = (KDA_RAW_INPUTS if raw_inputs else 0) | (KDA_UNBOUNDED_GATE if unbounded_gate else 0)
    if t.dtype == torch.bfloat16:
        return KDA_BF16 | flag
    if t.dtype == torch.float32:
        return KDA_F32 | flag
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _out(t, name, shape, dtype):
    """A caller-supplied output: the library writes through its bare pointer, so
    it must be a contiguous GPU tensor of exactly this shape and dtype."""
    if t is None:
        return None
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ws(t, name="workspace"):
    """A caller-supplied workspace: a contiguous GPU tensor (its byte size goes to
    the library, which checks it against what the call needs)."""
    if t is None or t is False:
        return t
    return _dev(t, name)


def _seqlens(cu_seqlens, cu_seqlens_host, T, device):
    """Return (device int32 tensor or None, host int32 numpy array or None, N)."""
    torch = _torch()
    if cu_seqlens is None and cu_seqlens_host is None:
        return None, None, 1
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.detach().to("cpu")
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host.numpy() if hasattr(cu_seqlens_host, "numpy")
                                           else cu_seqlens_host), dtype=np.int32)
    if cu_seqlens is None or not getattr(cu_seqlens, "is_cuda", False):
        cu_seqlens = torch.from_numpy(host).to(device)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    return cu_seqlens, host, int(host.shape[0] - 1)


def _prefill_common(q, k, v, g_logits, beta, A_log, initial_state, cu_seqlens, cu_seqlens_host):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("g_logits", g_logits), ("beta", beta)):
        _dev(t, name, q.dtype)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or g_logits.shape != (T, H, dk) or v.shape[:2] != (T, H) \
            or beta.shape != (T, H):
        raise ValueError("shape mismatch: q,k,g_logits [T,H,dk], v [T,H,dv], beta [T,H]")
    _dev(A_log, "A_log", torch.float32)
    cu_dev, cu_host, N = _seqlens(cu_seqlens, cu_seqlens_host, T, q.device)
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32)
        if tuple(initial_state.shape) != (N, H, dk, dv):
            raise ValueError(f"initial_state must be [{N},{H},{dk},{dv}]")
    return T, H, dk, dv, N, cu_dev, cu_host


def kda_chunk_fwd_workspace_size(N: int, T: int, H: int, dk: int = 128, dv: int = 128) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(N, T, H, dk, dv))


def kda_chunk_fwd(q, k, v, g_logits, beta, A_log=None, g_min: float = -5.0,
                  initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                  output_final_state: bool = True, compute: int = KDA_COMPUTE_AUTO,
                  o=None, final_state=None, workspace=None,
                  raw_inputs: bool = False,
                  unbounded_gate: bool = False) -> Tuple[object, Optional[object]]:
    """Chunkwise KDA prefill.  q, k, v, g_logits: [T, H, 128]; beta: [T, H] (same
    dtype, bf16 or fp32); A_log: [H] fp32 or None; initial_state: [N, H, 128, 128]
    fp32 or None; cu_seqlens: [N+1] int32 (device and/or host copy).
    workspace: None allocates one (uint8, kda_chunk_fwd_workspace_size bytes) when
    the two-kernel path applies (bf16 inputs, compute AUTO); False runs the fused
    single kernel; a uint8 device tensor is used as given.
    raw_inputs: q, k unnormalised and beta a logit (normalised and sigmoid in the
    kernels); unbounded_gate: g = -exp(A_h) softplus(z) instead of the bounded gate
    (g_min is then unused; the other prefill functions take both flags too).
    Returns (o [T, H, 128] in the input dtype, final_state [N, H, 128, 128] fp32 or None)."""
    torch = _torch()
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, v, g_logits, beta, A_log,
                                                       initial_state, cu_seqlens, cu_seqlens_host)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, H, dv), q.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if workspace is None:
        split = _dtype_code(q) == KDA_BF16 and int(compute) == KDA_COMPUTE_AUTO and T > 0
        workspace = (torch.empty(kda_chunk_fwd_workspace_size(N, T, H, dk, dv), dtype=torch.uint8,
                                 device=q.device) if split else False)
    _ws(workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is False else \
        (_ptr(workspace), workspace.numel() * workspace.element_size())
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(beta), _ptr(A_log),
                           float(g_min), _ptr(initial_state), _ptr(cu_dev), host_ptr, N, T, H,
                           dk, dv, _dtype_code(q, raw_inputs, unbounded_gate), int(compute),
                           _ptr(o), _ptr(final_state), ws_ptr, ws_bytes, _stream())
    _check(rc)
    return o, final_state


KDA_NOALLOC_SCRATCH_BYTES = 256 << 20  # kda_chunk_fwd_noalloc's device scratch


def kda_chunk_fwd_noalloc(q, k, v, g_logits, beta, A_log=None, g_min: float = -5.0,
                          initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                          output_final_state: bool = True, o=None, final_state=None,
                          raw_inputs: bool = False,
                          unbounded_gate: bool = False) -> Tuple[object, Optional[object]]:
    """``kda_chunk_fwd`` (two-kernel path, bf16) whose workspace is the library's
    static device scratch: the C call allocates nothing.  Sizes whose workspace
    exceeds KDA_NOALLOC_SCRATCH_BYTES raise KDAError (KDA_ERR_WORKSPACE).  Pass
    ``o`` (and ``final_state``) to allocate nothing here either.
    Returns (o, final_state) as ``kda_chunk_fwd``."""
    torch = _torch()
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, v, g_logits, beta, A_log,
                                                       initial_state, cu_seqlens, cu_seqlens_host)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, H, dv), q.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(beta),
                                   _ptr(A_log), float(g_min), _ptr(initial_state), _ptr(cu_dev),
                                   host_ptr, N, T, H, dk, dv,
                                   _dtype_code(q, raw_inputs, unbounded_gate), _ptr(o),
                                   _ptr(final_state), _stream())
    _check(rc)
    return o, final_state


def kda_chunk_fwd_unbounded(q, k, v, g_logits, beta, A_log=None, initial_state=None,
                            cu_seqlens=None, cu_seqlens_host=None,
                            output_final_state: bool = True, o=None, final_state=None,
                            workspace=None, raw_inputs: bool = False) -> Tuple[object, Optional[object]]:
    """``kda_chunk_fwd`` with the unbounded gate g = -exp(A_h) softplus(z).  bf16
    inputs run the two-kernel path with a workspace (None allocates one) or the
    fused kernel (``workspace=False``); fp32 inputs run the fused kernel in fp32
    arithmetic.  Returns (o, final_state) as ``kda_chunk_fwd``."""
    torch = _torch()
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, v, g_logits, beta, A_log,
                                                       initial_state, cu_seqlens, cu_seqlens_host)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, H, dv), q.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if workspace is None:
        workspace = torch.empty(max(1, kda_chunk_fwd_workspace_size(N, T, H, dk, dv)),
                                dtype=torch.uint8, device=q.device) \
            if _dtype_code(q) == KDA_BF16 else False
    _ws(workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is False else \
        (_ptr(workspace), workspace.numel() * workspace.element_size())
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_chunk_fwd_unbounded(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(beta),
                                     _ptr(A_log), _ptr(initial_state), _ptr(cu_dev), host_ptr, N,
                                     T, H, dk, dv, _dtype_code(q, raw_inputs), _ptr(o),
                                     _ptr(final_state), ws_ptr, ws_bytes, _stream())
    _check(rc)
    return o, final_state


def kda_checkpoint_count(N: int, T: int, interval: int) -> int:
    return int(load_library().kda_checkpoint_count(N, T, interval))


def checkpoint_index(cu_seqlens_host, d: int, j: int, interval: int) -> int:
    """Index in the checkpoint array of the state after the first j * interval
    tokens of document d (j >= 1, j * interval < the document's length)."""
    cpi = interval // 64
    first = int(cu_seqlens_host[d]) // 64 + d if cu_seqlens_host is not None else 0
    return (first + j * cpi - 1) // cpi


def kda_chunk_fwd_checkpoints(q, k, v, g_logits, beta, interval: int, A_log=None,
                              g_min: float = -5.0, initial_state=None, cu_seqlens=None,
                              cu_seqlens_host=None, output_final_state: bool = True, o=None,
                              final_state=None, checkpoints=None, workspace=None,
                              raw_inputs: bool = False, unbounded_gate: bool = False):
    """kda_chunk_fwd (two-kernel path, bf16) that also writes the state every
    ``interval`` tokens inside each document (see ``checkpoint_index``).
    Returns (o, final_state, checkpoints [kda_checkpoint_count, H, 128, 128] fp32)."""
    torch = _torch()
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, v, g_logits, beta, A_log,
                                                       initial_state, cu_seqlens, cu_seqlens_host)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, H, dv), q.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if checkpoints is None:
        n = kda_checkpoint_count(N, T, interval)
        checkpoints = torch.empty((max(n, 1), H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(kda_chunk_fwd_workspace_size(N, T, H, dk, dv), dtype=torch.uint8,
                                device=q.device)
    _ws(workspace)
    _dev(checkpoints, "checkpoints", torch.float32)  # its byte size is checked by the library
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_chunk_fwd_checkpoints(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(beta), _ptr(A_log), float(g_min),
        _ptr(initial_state), _ptr(cu_dev), host_ptr, N, T, H, dk, dv,
        _dtype_code(q, raw_inputs, unbounded_gate), int(interval), _ptr(checkpoints), checkpoints.numel() * checkpoints.element_size(),
        _ptr(o), _ptr(final_state), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream())
    _check(rc)
    return o, final_state, checkpoints


def kda_chunk_prep(q, k, g_logits, beta, workspace, A_log=None, g_min: float = -5.0,
                   cu_seqlens=None, cu_seqlens_host=None, raw_inputs: bool = False,
                   unbounded_gate: bool = False) -> None:
    """First half of the two-kernel prefill: writes every (head, chunk) image into
    ``workspace`` (uint8, kda_chunk_fwd_workspace_size bytes).  bf16 inputs only."""
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, q, g_logits, beta, A_log, None,
                                                       cu_seqlens, cu_seqlens_host)
    _ws(workspace)
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib.kda_chunk_prep(_ptr(q), _ptr(k), _ptr(g_logits), _ptr(beta), _ptr(A_log),
                              float(g_min), _ptr(cu_dev), host_ptr, N, T, H, dk, dv,
                              _dtype_code(q, raw_inputs, unbounded_gate), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream()))


def kda_chunk_recurrence(v, workspace, initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                         output_final_state: bool = True, o=None, final_state=None):
    """Second half of the two-kernel prefill: the chunk recurrence over the images
    kda_chunk_prep wrote.  Returns (o, final_state)."""
    torch = _torch()
    lib = load_library()
    _dev(v, "v")
    T, H, dv = v.shape
    dk = dv
    cu_dev, cu_host, N = _seqlens(cu_seqlens, cu_seqlens_host, T, v.device)
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32)
        if tuple(initial_state.shape) != (N, H, dk, dv):
            raise ValueError(f"initial_state must be [{N},{H},{dk},{dv}]")
    if o is None:
        o = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
    _out(o, "o", (T, H, dv), v.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    _ws(workspace)
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    _check(lib.kda_chunk_recurrence(_ptr(v), _ptr(initial_state), _ptr(cu_dev), host_ptr, N, T, H,
                                    dk, dv, _dtype_code(v), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(o),
                                    _ptr(final_state), _stream()))
    return o, final_state


def kda_segment_scan_workspace_size(N: int, T: int, H: int, n_segments: int = 0, dk: int = 128,
                                    dv: int = 128) -> int:
    return int(load_library().kda_segment_scan_workspace_size(N, T, H, n_segments, dk, dv))


def kda_default_segments() -> int:
    n = int(load_library().kda_default_segments())
    if n < 0:
        _check(n)
    return n


def kda_segment_scan(q, k, v, g_logits, beta, A_log=None, g_min: float = -5.0,
                     initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                     n_segments: int = 0, output_final_state: bool = True,
                     compute: int = KDA_COMPUTE_AUTO, workspace=None, o=None,
                     final_state=None, raw_inputs: bool = False, unbounded_gate: bool = False):
    """Prefill via per-segment affine pairs, an on-device pair scan and a re-run
    from exact entry states.  Same tensors as ``kda_chunk_fwd``; n_segments <= 0
    lets the library choose the count (bf16: one (segment, head) per compute unit
    while that is at most 32 segments; fp32: one segment per compute unit).
    Returns (o, final_state)."""
    torch = _torch()
    lib = load_library()
    T, H, dk, dv, N, cu_dev, cu_host = _prefill_common(q, k, v, g_logits, beta, A_log,
                                                       initial_state, cu_seqlens, cu_seqlens_host)
    n_seg = max(int(n_segments), 0)  # 0: the library's plan (see include/kda.h)
    need = kda_segment_scan_workspace_size(N, T, H, n_seg, dk, dv)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, H, dv), q.dtype)
    _out(final_state, "final_state", (N, H, dk, dv), torch.float32)
    _ws(workspace)
    host_ptr = None if cu_host is None else cu_host.ctypes.data_as(ctypes.c_void_p)
    rc = lib.kda_segment_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(beta), _ptr(A_log),
                              float(g_min), _ptr(initial_state), _ptr(cu_dev), host_ptr, N, T, H,
                              dk, dv, _dtype_code(q, raw_inputs, unbounded_gate), int(compute),
                              int(n_seg), _ptr(o),
                              _ptr(final_state), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream())
    _check(rc)
    return o, final_state


def _decode_common(state, cq, ck, cv, cz, cbeta, accepted, nq, nk, nv, nz, nbeta, A_log,
                   state_slots, err_flag):
    """Validate the decode tensors (device, dtype, contiguity, shapes); returns
    (N, H, d, W, S_pool)."""
    torch = _torch()
    _dev(state, "state", torch.float32)
    if nq.dim() != 3:
        raise ValueError("nq must be [N, H, 128]")
    N, H, d = nq.shape
    dt = nq.dtype
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, d, d):
        raise ValueError(f"state must be [S_pool, {H}, {d}, {d}], got {tuple(state.shape)}")
    S_pool = int(state.shape[0])
    for name, t in (("nk", nk), ("nv", nv), ("nz", nz)):
        _dev(t, name, dt)
        if tuple(t.shape) != (N, H, d):
            raise ValueError(f"{name} must be [{N}, {H}, {d}], got {tuple(t.shape)}")
    _dev(nq, "nq", dt)
    _dev(nbeta, "nbeta", dt)
    if tuple(nbeta.shape) != (N, H):
        raise ValueError(f"nbeta must be [{N}, {H}], got {tuple(nbeta.shape)}")
    W = 0
    if cq is not None:
        if cq.dim() != 4:
            raise ValueError("cq must be [N, W, H, 128]")
        W = int(cq.shape[1])
        for name, t in (("cq", cq), ("ck", ck), ("cv", cv), ("cz", cz)):
            _dev(t, name, dt)
            if t is None or tuple(t.shape) != (N, W, H, d):
                raise ValueError(f"{name} must be [{N}, {W}, {H}, {d}]")
        _dev(cbeta, "cbeta", dt)
        if cbeta is None or tuple(cbeta.shape) != (N, W, H):
            raise ValueError(f"cbeta must be [{N}, {W}, {H}]")
    _dev(accepted, "accepted", torch.int32)
    if accepted is None or tuple(accepted.shape) != (N,):
        raise ValueError(f"accepted must be [{N}] int32")
    _dev(state_slots, "state_slots", torch.int32)
    if state_slots is not None and tuple(state_slots.shape) != (N,):
        raise ValueError(f"state_slots must be [{N}] int32")
    if state_slots is None and S_pool < N:
        raise ValueError(f"state holds {S_pool} states but there are {N} sequences "
                         "(pass state_slots to map sequences into the pool)")
    _dev(A_log, "A_log", torch.float32)
    if A_log is not None and tuple(A_log.shape) != (H,):
        raise ValueError(f"A_log must be [{H}] float32")
    _dev(err_flag, "err_flag", torch.int32)
    if err_flag is not None and err_flag.numel() < 1:
        raise ValueError("err_flag must hold one int32")
    return N, H, d, W, S_pool


def kda_decode_step(state, cq, ck, cv, cz, cbeta, accepted, nq, nk, nv, nz, nbeta,
                    A_log=None, g_min: float = -5.0, state_slots=None, o=None, err_flag=None,
                    raw_inputs: bool = False, unbounded_gate: bool = False):
    """One decode step with speculative-verify replay, updating ``state`` in place.

    state: [S_pool, H, 128, 128] fp32; cq, ck, cv, cz: [N, W, H, 128]; cbeta: [N, W, H];
    accepted: [N] int32 (device); nq, nk, nv, nz: [N, H, 128]; nbeta: [N, H];
    state_slots: [N] int32 slots into the pool (None: sequence n uses state n).
    Slots outside the pool are skipped (outputs zero, err_flag bit
    KDA_DECODE_ERR_SLOT).  Returns o [N, H, 128] (output of the bonus token)."""
    torch = _torch()
    lib = load_library()
    N, H, d, W, S_pool = _decode_common(state, cq, ck, cv, cz, cbeta, accepted, nq, nk, nv, nz,
                                        nbeta, A_log, state_slots, err_flag)
    dt = nq.dtype
    if o is None:
        o = torch.empty((N, H, d), dtype=dt, device=nq.device)
    _out(o, "o", (N, H, d), dt)
    rc = lib.kda_decode_step(_ptr(state), S_pool, _ptr(state_slots), _ptr(cq), _ptr(ck), _ptr(cv),
                             _ptr(cz), _ptr(cbeta), _ptr(accepted), int(W), _ptr(nq), _ptr(nk),
                             _ptr(nv), _ptr(nz), _ptr(nbeta), _ptr(A_log), float(g_min), _ptr(o),
                             _ptr(err_flag), N, H, d, d, _dtype_code(nq, raw_inputs, unbounded_gate),
                             _stream())
    _check(rc)
    return o


def kda_decode_step_window(state, cq, ck, cv, cz, cbeta, accepted, nq, nk, nv, nz, nbeta,
                           wq, wk, wv, wz, wbeta, A_log=None, g_min: float = -5.0,
                           state_slots=None, o=None, o_window=None, err_flag=None,
                           raw_inputs: bool = False, unbounded_gate: bool = False):
    """``kda_decode_step`` followed, in the same kernel, by the next draft window.

    Arguments as for ``kda_decode_step`` plus wq, wk, wv, wz: [N, W2, H, 128] and
    wbeta: [N, W2, H], the drafts of the next window.  ``state`` receives the state
    after the bonus token, as with ``kda_decode_step``.  Returns (o, o_window):
    o [N, H, 128] for the bonus token, o_window [N, W2, H, 128] for the drafts."""
    torch = _torch()
    lib = load_library()
    N, H, d, W, S_pool = _decode_common(state, cq, ck, cv, cz, cbeta, accepted, nq, nk, nv, nz,
                                        nbeta, A_log, state_slots, err_flag)
    W2 = wq.shape[1]
    dt = nq.dtype
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv), ("wz", wz), ("wbeta", wbeta)):
        _dev(t, name, dt)
    for name, t in (("wk", wk), ("wv", wv), ("wz", wz)):
        if tuple(t.shape) != tuple(wq.shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(wq.shape)}")
    if tuple(wq.shape) != (N, W2, H, d) or tuple(wbeta.shape) != (N, W2, H):
        raise ValueError("next-window inputs must be [N, W2, H, 128] and [N, W2, H]")
    if o is None:
        o = torch.empty((N, H, d), dtype=dt, device=nq.device)
    if o_window is None:
        o_window = torch.empty((N, W2, H, d), dtype=dt, device=nq.device)
    _out(o_window, "o_window", (N, W2, H, d), dt)
    _out(o, "o", (N, H, d), dt)
    rc = lib.kda_decode_step_window(
        _ptr(state), S_pool, _ptr(state_slots), _ptr(cq), _ptr(ck), _ptr(cv), _ptr(cz), _ptr(cbeta),
        _ptr(accepted), int(W), _ptr(nq), _ptr(nk), _ptr(nv), _ptr(nz), _ptr(nbeta), _ptr(wq),
        _ptr(wk), _ptr(wv), _ptr(wz), _ptr(wbeta), int(W2), _ptr(A_log), float(g_min), _ptr(o),
        _ptr(o_window), _ptr(err_flag), N, H, d, d, _dtype_code(nq, raw_inputs, unbounded_gate),
        _stream())
    _check(rc)
    return o, o_window


__all__ = ["KDA_RAW_INPUTS", "kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_segment_scan", "kda_segment_scan_workspace_size",
           "kda_default_segments", "kda_decode_step", "kda_decode_step_window",
           "kda_chunk_fwd_unbounded", "kda_chunk_fwd_checkpoints", "kda_checkpoint_count", "load_library", "KDAError",
           "KDA_COMPUTE_AUTO", "KDA_COMPUTE_F32"]
