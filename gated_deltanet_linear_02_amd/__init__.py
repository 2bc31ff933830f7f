"""Gated DeltaNet layer on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libgdn.so`` (the C ABI in ``include/gdn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals torch tensors (device memory) and the current HIP stream into
the C calls, and turns status codes into exceptions. If the library has not
been built, importing works but every call raises.

Entry points (same names as the C ABI, without the ``gdn_`` prefix):
    prefill(q, k, v, g, beta, cu_seqlens, ...)  -> (out, final_state)
    decode_step(q, k, v, g, beta, state, ...)   -> out
    (bf16 state tensors, or ``norm_weight=``, call gdn_prefill_ex /
    gdn_decode_step_ex: states stored in bf16 with fp32 arithmetic, and the
    output rows RMS-normalised, times one weight per value channel)
    prefill_workspace_size(...)
    prefill_noalloc(q, k, v, g, beta, cu_seqlens, out=, final_state=, ...)
        -> gdn_prefill_noalloc: the workspace is the library's own fixed
        device array (nothing is allocated; out and states must be given)
    tune_prefill(q, k, v, g, beta, cu_seqlens, ...) -> chosen method, per-candidate
        times and gate errors (cached for prefill's chunk 0);
    tune_cache_clear / tune_cache_size / tune_cache_save / tune_cache_load
    timing_start(max_launches) / timing_stop()  -> per-kernel launch times
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

import torch

__all__ = [
    "GdnError", "lib_path", "load", "prefill", "prefill_noalloc", "decode_step", "prefill_workspace_size", "prefill_method",
    "prefill_plan", "tune_prefill", "method_name", "TUNE_CANDIDATES", "tune_cache_clear", "tune_cache_size",
    "tune_cache_save", "tune_cache_load", "timing_start", "timing_stop", "abi_version", "KERNEL_KINDS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdn.so")
_lib = None
_lock = threading.Lock()

GDN_BF16, GDN_F32 = 0, 1
KERNEL_KINDS = ("schedule", "prep", "scan", "decode", "token_scan", "decode_norm", "norm_apply")

STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL_ARG", 2: "GDN_ERR_BAD_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
    4: "GDN_ERR_WORKSPACE", 5: "GDN_ERR_HIP", 6: "GDN_ERR_ALIAS", 7: "GDN_ERR_BAD_VALUE",
    8: "GDN_ERR_MISALIGNED",
}


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdn.so (built by ``python -m gated_deltanet_linear_02_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m gated_deltanet_linear_02_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.gdn_abi_version.restype = i32
        L.gdn_abi_version.argtypes = []
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [i32]
        L.gdn_prefill_workspace_size.restype = sz
        L.gdn_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32]
        L.gdn_prefill_method.restype = i32
        L.gdn_prefill_method.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
        L.gdn_prefill_method_hint.restype = i32
        L.gdn_prefill_method_hint.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(i32)]
        L.gdn_prefill_hint.restype = i32
        L.gdn_prefill_hint.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32,
                                       f32, i32, i32, vp, vp, i32, vp, f32, vp, vp, sz, vp]
        L.gdn_prefill.restype = i32
        L.gdn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                  f32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.gdn_prefill_noalloc.restype = i32
        L.gdn_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                          f32, i32, i32, vp, vp, vp, vp]
        L.gdn_prefill_ex.restype = i32
        L.gdn_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                     f32, i32, i32, vp, vp, i32, vp, f32, vp, vp, sz, vp]
        L.gdn_decode_step.restype = i32
        L.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                      vp, vp, i32, vp, vp]
        L.gdn_decode_step_ex.restype = i32
        L.gdn_decode_step_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                         vp, i32, vp, i32, vp, f32, vp, vp]
        L.gdn_tune_prefill_scratch_size.restype = sz
        L.gdn_tune_prefill_scratch_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
        L.gdn_tune_prefill.restype = i32
        L.gdn_tune_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, f32, i32, i32,
                                       vp, f32, vp, sz, vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(f32), ctypes.POINTER(f32)]
        L.gdn_tune_cache_clear.restype = None
        L.gdn_tune_cache_clear.argtypes = []
        L.gdn_tune_cache_size.restype = i32
        L.gdn_tune_cache_size.argtypes = []
        L.gdn_tune_cache_save.restype = i32
        L.gdn_tune_cache_save.argtypes = [ctypes.c_char_p]
        L.gdn_tune_cache_load.restype = i32
        L.gdn_tune_cache_load.argtypes = [ctypes.c_char_p, ctypes.POINTER(i32)]
        L.gdn_timing_start.restype = i32
        L.gdn_timing_start.argtypes = [i32]
        L.gdn_timing_stop.restype = i32
        L.gdn_timing_stop.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(f32), i32]
        _lib = L
        return _lib


def _check(status: int):
    if status != 0:
        msg = load().gdn_status_string(status).decode()
        raise GdnError(status, msg)


def abi_version() -> int:
    return int(load().gdn_abi_version())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GDN_BF16
    if t == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgdn must be contiguous")
    return t.data_ptr() or None


def _stream(device: torch.device, stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream or None


def _check_norm_weight(w: torch.Tensor, dv: int) -> None:
    if w.dtype != torch.float32 or w.numel() != dv:
        raise TypeError(f"norm_weight must be float32 with {dv} entries")


def _expect(name: str, t: Optional[torch.Tensor], shape: tuple, dtype: Optional[torch.dtype] = None) -> None:
    """The library reads and writes tensors by their declared sizes alone, so
    a smaller tensor than the call implies would be accessed past its end:
    shapes and dtypes are checked here, before the call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}, expected {dtype}")


def _on_device(dev: torch.device, **tensors) -> None:
    """Every tensor handed to the library must live on the GPU the call runs
    on: a host pointer would be dereferenced by a kernel."""
    for name, t in tensors.items():
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def prefill_workspace_size(num_seqs: int, total_tokens: int, hk: int, hv: int, dk: int, dv: int,
                           chunk: int, io_dtype: torch.dtype) -> int:
    return int(load().gdn_prefill_workspace_size(num_seqs, total_tokens, hk, hv, dk, dv, chunk,
                                                 _dtype_code(io_dtype)))


def prefill_plan(num_seqs: int, total_tokens: int, hk: int, hv: int, d: int, chunk: int = 0,
                 io_dtype: torch.dtype = torch.bfloat16, gate_dtype: torch.dtype = torch.float32,
                 max_seqlen: Optional[int] = None) -> Tuple[int, int]:
    """The method ``prefill`` uses for these sizes (``gdn_prefill_method``,
    or ``gdn_prefill_method_hint`` with ``max_seqlen``, the longest
    sequence's length): (chunk, rows) with chunk 1 (token by token), 16, 32
    or 64 and rows the chunked scan's state rows per workgroup (16, 32, 64 or
    128; 0 token by token); (0, 0) if the sizes are rejected."""
    rows = ctypes.c_int32(0)
    c = load().gdn_prefill_method_hint(num_seqs, total_tokens, int(max_seqlen or 0), hk, hv, d, d, chunk,
                                       _dtype_code(io_dtype), _dtype_code(gate_dtype), ctypes.byref(rows))
    return int(c), int(rows.value)


def prefill_method(num_seqs: int, total_tokens: int, hk: int, hv: int, d: int, chunk: int = 0,
                   io_dtype: torch.dtype = torch.bfloat16, gate_dtype: torch.dtype = torch.float32) -> int:
    """The chunk of ``prefill_plan``: 1 (token by token), 16, 32 or 64; 0 if
    the sizes are rejected."""
    return prefill_plan(num_seqs, total_tokens, hk, hv, d, chunk, io_dtype, gate_dtype)[0]


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
            cu_seqlens: torch.Tensor, *, chunk: int = 0, scale: float = 1.0,
            initial_state: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            write_final_state: bool = True, norm_weight: Optional[torch.Tensor] = None,
            norm_eps: float = 1e-6, state_dtype: Optional[torch.dtype] = None,
            max_seqlen: Optional[int] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill over packed sequences (``gdn_prefill``).

    q, k [T, hk, dk]; v [T, hv, dv] (bf16 or fp32, one dtype); g, beta [T, hv]
    (bf16 or fp32); cu_seqlens int32 [N + 1] on the device; states fp32
    [N, hv, dv, dk]. ``final_state`` may be ``initial_state`` (in place).
    ``chunk``: 16, 32 or 64 (chunked), 1 (token by token) or 0 (the tuned
    choice for the shape, else a rule by mean sequence length; see
    ``prefill_method``).
    ``norm_weight`` (fp32 [dv], or None): RMS-normalise every output row,
    y = o * w / sqrt(mean(o^2) + norm_eps).
    States are fp32 or bf16 (``gdn_prefill_ex``): the dtype of the state
    tensors given, else ``state_dtype`` (default fp32).
    ``max_seqlen`` (host int, or None): the longest sequence's length, a hint
    for the method rule on uneven batches (``gdn_prefill_hint``).
    Missing out / final_state / workspace are allocated with torch.
    """
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d int32 tensor")
    io = _dtype_code(q.dtype)
    gate = _dtype_code(g.dtype)
    _expect("k", k, (T, hk, dk), q.dtype)
    _expect("v", v, (T, hv, dv), q.dtype)
    _expect("g", g, (T, hv))
    _expect("beta", beta, (T, hv), g.dtype)
    _expect("out", out, (T, hv, dv), q.dtype)
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        _expect(name, st, (N, hv, dv, dk))
    dev = q.device
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=dev)
    given = {t.dtype for t in (initial_state, final_state) if t is not None}
    if len(given) > 1:
        raise TypeError("initial_state and final_state must have one dtype")
    sdt = given.pop() if given else (state_dtype or torch.float32)
    if state_dtype is not None and sdt != state_dtype:
        raise TypeError(f"state tensors are {sdt}, state_dtype says {state_dtype}")
    if final_state is None and write_final_state:
        final_state = torch.empty((N, hv, dv, dk), dtype=sdt, device=dev)
    need = prefill_workspace_size(N, T, hk, hv, dk, dv, chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _on_device(dev, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, initial_state=initial_state,
               final_state=final_state, out=out, workspace=workspace, norm_weight=norm_weight)
    ws_bytes = workspace.numel() * workspace.element_size()
    if max_seqlen is not None:
        if norm_weight is not None:
            _check_norm_weight(norm_weight, dv)
        status = load().gdn_prefill_hint(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, int(max_seqlen),
            hk, hv, dk, dv, chunk, float(scale), io, gate,
            _ptr(initial_state), _ptr(final_state), _dtype_code(sdt), _ptr(norm_weight), float(norm_eps),
            _ptr(out), _ptr(workspace), ws_bytes, _stream(dev, stream))
    elif norm_weight is None and sdt == torch.float32:
        status = load().gdn_prefill(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
            hk, hv, dk, dv, chunk, float(scale), io, gate,
            _ptr(initial_state), _ptr(final_state), _ptr(out),
            _ptr(workspace), ws_bytes, _stream(dev, stream))
    else:
        if norm_weight is not None:
            _check_norm_weight(norm_weight, dv)
        status = load().gdn_prefill_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
            hk, hv, dk, dv, chunk, float(scale), io, gate,
            _ptr(initial_state), _ptr(final_state), _dtype_code(sdt), _ptr(norm_weight), float(norm_eps),
            _ptr(out), _ptr(workspace), ws_bytes, _stream(dev, stream))
    _check(status)
    return out, final_state


def prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                    cu_seqlens: torch.Tensor, *, out: torch.Tensor, final_state: Optional[torch.Tensor] = None,
                    initial_state: Optional[torch.Tensor] = None, chunk: int = 0, scale: float = 1.0,
                    stream=None) -> None:
    """``gdn_prefill_noalloc``: ``prefill`` with fp32 states and no
    normalisation, using the library's fixed device workspace
    (GDN_NOALLOC_SCRATCH_BYTES per GPU) instead of one from the caller.
    Nothing is allocated here either: ``out`` must be given, and the final
    state is written only if ``final_state`` is. Calls that may overlap on one
    GPU share that workspace and must be serialised by the caller."""
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d int32 tensor")
    _expect("k", k, (T, hk, dk), q.dtype)
    _expect("v", v, (T, hv, dv), q.dtype)
    _expect("g", g, (T, hv))
    _expect("beta", beta, (T, hv), g.dtype)
    _expect("out", out, (T, hv, dv), q.dtype)
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        _expect(name, st, (N, hv, dv, dk), torch.float32)
    dev = q.device
    _on_device(dev, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, initial_state=initial_state,
               final_state=final_state, out=out)
    _check(load().gdn_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
        hk, hv, dk, dv, chunk, float(scale), _dtype_code(q.dtype), _dtype_code(g.dtype),
        _ptr(initial_state), _ptr(final_state), _ptr(out), _stream(dev, stream)))


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                state: torch.Tensor, *, scale: float = 1.0, state_slots: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                norm_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """One token per sequence against resident fp32 states, updated in place
    (``gdn_decode_step``). q, k [B, hk, dk]; v [B, hv, dv]; g, beta [B, hv];
    state [slots, hv, dv, dk]; state_slots int32 [B] on the device or None.
    ``norm_weight`` (fp32 [dv], or None): the output rows RMS-normalised in
    the same kernel. A bf16 ``state`` is stored in bf16 between steps, with
    fp32 arithmetic (``gdn_decode_step_ex``)."""
    B, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if state.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("state must be float32 or bfloat16")
    _expect("k", k, (B, hk, dk), q.dtype)
    _expect("v", v, (B, hv, dv), q.dtype)
    _expect("g", g, (B, hv))
    _expect("beta", beta, (B, hv), g.dtype)
    _expect("out", out, (B, hv, dv), q.dtype)
    _expect("state", state, (state.shape[0], hv, dv, dk))
    _expect("state_slots", state_slots, (B,))
    if state_slots is not None and state_slots.dtype != torch.int32:
        raise TypeError("state_slots must be int32")
    if out is None:
        out = torch.empty((B, hv, dv), dtype=q.dtype, device=q.device)
    _on_device(q.device, k=k, v=v, g=g, beta=beta, state=state, state_slots=state_slots, out=out,
               norm_weight=norm_weight)
    if norm_weight is None and state.dtype == torch.float32:
        status = load().gdn_decode_step(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, hk, hv, dk, dv, float(scale),
            _dtype_code(q.dtype), _dtype_code(g.dtype), _ptr(state), _ptr(state_slots),
            state.shape[0], _ptr(out), _stream(q.device, stream))
    else:
        if norm_weight is not None:
            _check_norm_weight(norm_weight, dv)
        status = load().gdn_decode_step_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, hk, hv, dk, dv, float(scale),
            _dtype_code(q.dtype), _dtype_code(g.dtype), _ptr(state), _dtype_code(state.dtype),
            _ptr(state_slots), state.shape[0], _ptr(norm_weight), float(norm_eps), _ptr(out),
            _stream(q.device, stream))
    _check(status)
    return out


# gdn_tune_prefill's candidates in its order: (chunk, state rows per scan
# workgroup), named "chunk/rows" ("1" token by token).
TUNE_CANDIDATES = ((64, 16), (64, 32), (64, 64), (64, 128), (32, 16), (32, 32), (32, 64), (32, 128),
                   (16, 16), (16, 32), (16, 64), (16, 128), (1, 0))


def method_name(chunk: int, rows: int) -> str:
    return "1" if chunk == 1 else f"{chunk}/{rows}"


def tune_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                 cu_seqlens: torch.Tensor, *, scale: float = 1.0, initial_state: Optional[torch.Tensor] = None,
                 gate_tol: float = 1.0 / 64, scratch: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Measure every prefill method on these inputs (``gdn_tune_prefill``):
    methods whose output or final state differs from chunk 64's (16 rows) by
    more than gate_tol of the largest magnitude are rejected, the fastest of
    the rest is returned and cached for ``prefill(chunk=0)`` on this device
    and shape bucket. Returns {"chunk": c, "rows": r, "method": name,
    "ms": {name: t}, "err": {name: e}}, names as ``method_name`` (t = -1 when
    rejected or not applicable, e = -1 when not run). Synchronises the
    stream."""
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise TypeError("cu_seqlens must be a 1-d int32 tensor")
    _expect("k", k, (T, hk, dk), q.dtype)
    _expect("v", v, (T, hv, dv), q.dtype)
    _expect("g", g, (T, hv))
    _expect("beta", beta, (T, hv), g.dtype)
    _expect("initial_state", initial_state, (N, hv, dv, dk))
    dev = q.device
    need = int(load().gdn_tune_prefill_scratch_size(N, T, hk, hv, dk, dv, _dtype_code(q.dtype)))
    if need == 0:
        raise GdnError(2, "shape rejected")
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    _on_device(dev, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, initial_state=initial_state,
               scratch=scratch)
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("tuning takes an fp32 initial state")
    chosen = ctypes.c_int32(0)
    rows = ctypes.c_int32(0)
    n = len(TUNE_CANDIDATES)
    ms = (ctypes.c_float * n)()
    err = (ctypes.c_float * n)()
    _check(load().gdn_tune_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, hk, hv, dk, dv, float(scale),
        _dtype_code(q.dtype), _dtype_code(g.dtype), _ptr(initial_state), float(gate_tol), _ptr(scratch),
        scratch.numel() * scratch.element_size(), _stream(dev, stream), ctypes.byref(chosen), ctypes.byref(rows),
        ms, err))
    names = [method_name(c, r) for c, r in TUNE_CANDIDATES]
    return {"chunk": int(chosen.value), "rows": int(rows.value),
            "method": method_name(int(chosen.value), int(rows.value)),
            "ms": {nm: float(ms[i]) for i, nm in enumerate(names)},
            "err": {nm: float(err[i]) for i, nm in enumerate(names)}}


def tune_cache_clear() -> None:
    load().gdn_tune_cache_clear()


def tune_cache_size() -> int:
    return int(load().gdn_tune_cache_size())


def tune_cache_save(path: str) -> None:
    _check(load().gdn_tune_cache_save(os.fsencode(path)))


def tune_cache_load(path: str) -> int:
    n = ctypes.c_int32(0)
    _check(load().gdn_tune_cache_load(os.fsencode(path), ctypes.byref(n)))
    return int(n.value)


def timing_start(max_launches: int) -> None:
    """Bracket the library's next ``max_launches`` kernel launches with HIP events."""
    _check(load().gdn_timing_start(max_launches))


def timing_stop() -> Dict[str, Dict[str, float]]:
    """Wait for the timed launches; per kernel kind: launch count, total and mean ms."""
    n = len(KERNEL_KINDS)
    counts = (ctypes.c_int32 * n)()
    ms = (ctypes.c_float * n)()
    _check(load().gdn_timing_stop(counts, ms, n))
    res = {}
    for i, name in enumerate(KERNEL_KINDS):
        c = int(counts[i])
        res[name] = {"count": c, "total_ms": float(ms[i]), "mean_ms": float(ms[i]) / c if c else 0.0}
    return res
