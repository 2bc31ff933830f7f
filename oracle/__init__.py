"""CPU oracle for the Gated DeltaNet layer (float64).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The product path (the HIP library and its
binding) never imports this package, and this package never imports the
product path.

What is here:

* ``scan``          -- the plain definition, token by token, in C
                       (``gdn_oracle.c``), threaded over (sequence, value head).
* ``decode_step``   -- the same definition for one token per sequence,
                       continuing from given states.
* ``literal_scan``  -- the recurrence written with explicit matrices,
                       ``S <- a S (I - b k k^T) + b v k^T``, in numpy; tiny
                       inputs only.
* ``chunked``       -- the chunk-parallel evaluation of the same recurrence
                       (the reorganisation into blocks that expose matrix
                       products, "Optimiser l'inference sur appareil pour Apple
                       Silicon", section "Qwen cree trois formes de charges de
                       travail distinctes"), written from its derivation in
                       numpy float64; used only to brute-force "scan ==
                       chunked" on tiny inputs.
* ``rms_norm``      -- the output normalisation that follows the recurrent
                       update (section "Reduire le trafic intermediaire et
                       d'etat" fuses the update with a normalisation
                       without giving its form): per (token, value head),
                       the dv outputs divided by their root mean square,
                       with eps inside the root, times one weight per value
                       channel shared by all heads.

* ``round_to_bf16`` -- rounding of float64 values to the nearest bfloat16
                       (ties to even), for states stored in bf16 between
                       calls: the storage variant whose accuracy the pages
                       argue about (fp32 states in "Maintenir l'etat
                       recurrent sur la puce" of "Optimiser l'inference
                       sur appareil pour Apple Silicon", bf16 recurrence
                       states in the engine of "On descend d'un cran : #004
                       le meme compilateur sur les puces d'Apple").

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, scalar cases worked
by hand and cross-form brute force).

Conventions (readings where the pages are silent):
* value head h uses query/key head h // (hv // hk);
* g is the log of the decay a (a = exp(g)), b is used as given;
* layouts are token-major: q, k [T, hk, dk], v/out [T, hv, dv],
  g/beta [T, hv]; states [N, hv, dv, dk] with S[i][j], i over values.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            d = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.gdn_oracle_scan.restype = ctypes.c_int
            lib.gdn_oracle_scan.argtypes = [
                d, d, d, d, d, ctypes.POINTER(ctypes.c_int64), i64,
                i64, i64, i64, i64, ctypes.c_double,
                d, d, d, ctypes.POINTER(ctypes.c_int64), i64, ctypes.c_int]
            _lib = lib
    return _lib


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def scan(q, k, v, g, beta, cu_seqlens, *, scale: float = 1.0,
         initial_state=None, heads: Optional[Sequence[int]] = None,
         threads: Optional[int] = None, out=None, final_state=None
         ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 scan over packed sequences.

    Returns (out [T, hv, dv], final_state [N, hv, dv, dk]). With ``heads``,
    only those value heads are computed; the rest of ``out``/``final_state``
    stay zero (or keep what the caller passed in).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, hv) or beta.shape != (T, hv):
        raise ValueError("inconsistent input shapes")
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0 and end at T")
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        if s0.shape != (N, hv, dv, dk):
            raise ValueError("initial_state shape")
    if out is None:
        out = np.zeros((T, hv, dv), dtype=np.float64)
    if final_state is None:
        final_state = np.zeros((N, hv, dv, dk), dtype=np.float64)
    h_arr = None
    n_heads = 0
    if heads is not None:
        h_arr = np.ascontiguousarray(heads, dtype=np.int64)
        n_heads = len(h_arr)
    rc = lib.gdn_oracle_scan(
        _dptr(q), _dptr(k), _dptr(v), _dptr(g), _dptr(beta),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
        hk, hv, dk, dv, float(scale), _dptr(s0), _dptr(out), _dptr(final_state),
        None if h_arr is None else h_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        n_heads, int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_scan failed with code {rc}")
    return out, final_state


def decode_step(q, k, v, g, beta, state, *, scale: float = 1.0,
                threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One token per sequence: q, k [B, hk, dk], v [B, hv, dv], g/beta [B, hv],
    state [B, hv, dv, dk]. Returns (out [B, hv, dv], new_state)."""
    B = np.asarray(q).shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    return scan(q, k, v, g, beta, cu, scale=scale, initial_state=state, threads=threads)


def literal_scan(q, k, v, g, beta, cu_seqlens, *, scale: float = 1.0,
                 initial_state=None) -> Tuple[np.ndarray, np.ndarray]:
    """The recurrence with explicit matrices (tiny inputs):
    S <- exp(g) S (I - b k k^T) + b v k^T,  o = scale S q."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    N = len(cu) - 1
    out = np.zeros((T, hv, dv))
    fin = np.zeros((N, hv, dv, dk))
    eye = np.eye(dk)
    for n in range(N):
        for h in range(hv):
            S = np.zeros((dv, dk)) if initial_state is None else \
                np.array(initial_state[n, h], dtype=np.float64)
            for t in range(cu[n], cu[n + 1]):
                kk = k[t, h // grp][:, None]
                vv = v[t, h][:, None]
                a = np.exp(g[t, h])
                b = beta[t, h]
                S = a * (S @ (eye - b * (kk @ kk.T))) + b * (vv @ kk.T)
                out[t, h] = scale * (S @ q[t, h // grp])
            fin[n, h] = S
    return out, fin


def chunked(q, k, v, g, beta, cu_seqlens, *, chunk: int, scale: float = 1.0,
            initial_state=None) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk-parallel evaluation (WY / UT form), numpy float64.

    Within a chunk of C tokens starting from state S0, with cumulative
    log-decay c_t = sum_{s<=t} g_s and gamma_t = exp(c_t):
      A[t, s] = b_t exp(c_t - c_s) (k_t . k_s)          for s < t, else 0
      U = (I + A)^{-1} (diag(b) V - diag(b gamma) K S0^T)  rows are u_t
      O = scale (diag(gamma) Q S0^T + M U),   M[t, s] = exp(c_t - c_s)(q_t . k_s), s <= t
      S_end = gamma_C S0 + U^T diag(exp(c_C - c)) K
    The last chunk of a sequence may be shorter than `chunk`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    N = len(cu) - 1
    out = np.zeros((T, hv, dv))
    fin = np.zeros((N, hv, dv, dk))
    for n in range(N):
        for h in range(hv):
            S = np.zeros((dv, dk)) if initial_state is None else \
                np.array(initial_state[n, h], dtype=np.float64)
            for t0 in range(cu[n], cu[n + 1], chunk):
                t1 = min(t0 + chunk, cu[n + 1])
                K = k[t0:t1, h // grp]
                Q = q[t0:t1, h // grp]
                V = v[t0:t1, h]
                b = beta[t0:t1, h]
                c = np.cumsum(g[t0:t1, h])
                gam = np.exp(c)
                diff = c[:, None] - c[None, :]
                low_strict = np.tril(np.ones((t1 - t0, t1 - t0)), -1)
                low_incl = np.tril(np.ones((t1 - t0, t1 - t0)), 0)
                # exp only where the mask keeps the entry (the masked-out
                # upper triangle could overflow)
                decay_strict = np.where(low_strict > 0, np.exp(np.where(low_strict > 0, diff, 0.0)), 0.0)
                decay_incl = np.where(low_incl > 0, np.exp(np.where(low_incl > 0, diff, 0.0)), 0.0)
                A = b[:, None] * decay_strict * (K @ K.T)
                rhs = b[:, None] * V - (b * gam)[:, None] * (K @ S.T)
                U = np.linalg.solve(np.eye(t1 - t0) + A, rhs)
                M = decay_incl * (Q @ K.T)
                out[t0:t1, h] = scale * (gam[:, None] * (Q @ S.T) + M @ U)
                tail = np.exp(c[-1] - c)
                S = gam[-1] * S + U.T @ (tail[:, None] * K)
            fin[n, h] = S
    return out, fin


def rms_norm(o, weight, eps: float) -> np.ndarray:
    """Output normalisation over the last axis, float64:
    y[..., i] = o[..., i] * weight[i] / sqrt(mean_j o[..., j]^2 + eps).

    ``o`` is [..., dv] (the layer outputs, one row per token and value head),
    ``weight`` [dv]. With eps = 0 an all-zero row gives NaN (0/0), as the
    definition does."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (o.shape[-1],):
        raise ValueError("weight must have one entry per value channel")
    if not (eps >= 0.0):
        raise ValueError("eps must be >= 0")
    mean_sq = np.mean(o * o, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return o / np.sqrt(mean_sq + float(eps)) * w


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant
    bits, the exponent range of float32), ties to even; returned as float64.
    Overflow goes to +-inf, NaN stays NaN. Written from the definition:
    scale by a power of two so that the representable neighbours are
    consecutive integers, then round half to even (numpy's rint)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    ax = np.abs(x[fin])
    # exponent e with 2^e <= |x| < 2^(e+1); below 2^-126 the spacing stays
    # that of the smallest normal exponent (subnormals)
    e = np.maximum(np.floor(np.log2(ax)), -126.0)
    # guard the floor of log2 against rounding at exact powers of two
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, -126.0)
    ulp_exp = (e - 7).astype(np.int64)  # 7 fraction bits
    r = np.ldexp(np.rint(np.ldexp(ax, -ulp_exp)), ulp_exp)
    r = np.where(r >= 2.0 ** 128, np.inf, r)  # past the largest finite bf16 (rounded up into 2^128)
    out[fin] = np.sign(x[fin]) * r
    return out
