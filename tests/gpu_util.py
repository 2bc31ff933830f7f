"""Shared helpers for the GPU parity tests (not collected by pytest)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle

# Tolerances: max |gpu - ref| / max |ref| over the compared tensor.
TOL_BF16 = 2e-2   # bf16 outputs (and bf16-mode final states)
TOL_F32 = 1e-4    # fp32 I/O mode: outputs and final states


def gpu_available() -> bool:
    return torch.cuda.device_count() > 0


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")


def note(msg: str) -> None:
    """Print (and flush) what the next GPU step is, so a fault names its case."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_torch(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def device_inputs(inp: gs.GdnInputs, device="cuda") -> dict:
    d = dict(
        q=to_torch(inp.q, inp.io_dtype, device), k=to_torch(inp.k, inp.io_dtype, device),
        v=to_torch(inp.v, inp.io_dtype, device), g=to_torch(inp.g, inp.gate_dtype, device),
        beta=to_torch(inp.beta, inp.gate_dtype, device),
        cu_seqlens=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device),
    )
    d["initial_state"] = None if inp.initial_state is None else \
        torch.from_numpy(inp.initial_state).to(device)
    return d


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    if den == 0.0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max()) / den


def oracle_ref(inp: gs.GdnInputs, *, heads=None, scale=1.0, initial_state=None):
    w = inp.widened()
    s0 = w["initial_state"] if initial_state is None else initial_state
    return oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"],
                       scale=scale, initial_state=s0, heads=heads)


def run_prefill(inp: gs.GdnInputs, *, chunk: int, scale=1.0, nan_fill=True, **kw):
    d = device_inputs(inp)
    T, hv, dv = inp.total_tokens, inp.hv, inp.dv
    out_dtype = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    out = torch.full((T, hv, dv), float("nan") if nan_fill else 0.0, dtype=out_dtype, device="cuda")
    fin = torch.full((inp.num_seqs, hv, dv, inp.dk), float("nan"), dtype=torch.float32, device="cuda")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                       scale=scale, initial_state=d["initial_state"], final_state=fin, out=out, **kw)
    torch.cuda.synchronize()
    return o, f


def tol(io_dtype: str) -> float:
    return TOL_BF16 if io_dtype == "bf16" else TOL_F32
