"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle. It draws random numbers and rounds them to the storage formats; it
contains none of the recurrence's arithmetic.

Workload shapes follow the Qwen hybrid models described in "Optimiser
l'inference sur appareil pour Apple Silicon", section "Qwen cree trois formes
de charges de travail distinctes" (Gated DeltaNet layers with a fixed-size
recurrent state per head): 16 query/key heads shared by 32 value heads with
head dimension 128. The value distributions are:

* q, k ~ N(0, 1), L2-normalised per (token, head) in float64;
* v ~ N(0, 1);
* log-decay g = log a = -softplus(x), x ~ N(-1, 1);
* write strength b = sigmoid(x), x ~ N(0, 1);
* initial states ~ N(0, 0.02**2) (standard deviation 0.02);
* output-normalisation weights (one per value channel) ~ U(0.5, 1.5), the
  pages giving no trained values.

Storage rounding: values are made in float64, rounded to float32 with
round-to-nearest-even (numpy's cast) and, for bf16 storage, rounded again
from float32 to bfloat16 with round-to-nearest-even. bf16 tensors are carried
as uint16 bit patterns so that both sides see identical bits.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

SEED_BASE = 20261202


# --------------------------------------------------------------------------
# bfloat16 storage helpers (round-to-nearest-even, bit exact)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to a quiet NaN; infinities are preserved. Finite values
    whose rounding overflows become +-inf, as IEEE rounding requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # Only NaN bit patterns can wrap around in 32 bits; they are replaced below.
    with np.errstate(over="ignore"):
        rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    is_nan = np.isnan(x)
    if is_nan.any():
        out = np.where(is_nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16), out)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to a storage dtype: 'bf16' -> uint16 bits, 'f32' -> float32."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return x32
    raise ValueError(f"unknown storage dtype {dtype!r}")


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# Random draws
# --------------------------------------------------------------------------

def _unit_rows(rng: np.random.Generator, shape: Sequence[int]) -> np.ndarray:
    x = rng.standard_normal(size=tuple(shape))
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0.0] = 1.0
    return x / n


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    # -log(1 + e^x), evaluated without overflow.
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclasses.dataclass
class GdnInputs:
    """One packed batch of layer inputs in storage formats.

    Shapes (T = total tokens, N = sequences):
      q, k: [T, HK, dk]; v: [T, HV, dv]; g, beta: [T, HV];
      cu_seqlens: int32 [N + 1]; initial_state: float32 [N, HV, dv, dk] or None.
    io_dtype / gate_dtype are 'bf16' (uint16 bits) or 'f32'.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    initial_state: Optional[np.ndarray]
    hk: int
    hv: int
    dk: int
    dv: int
    io_dtype: str
    gate_dtype: str

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    def widened(self):
        """float64 copies of every input, exactly equal to the stored values."""
        return dict(
            q=widen(self.q, self.io_dtype),
            k=widen(self.k, self.io_dtype),
            v=widen(self.v, self.io_dtype),
            g=widen(self.g, self.gate_dtype),
            beta=widen(self.beta, self.gate_dtype),
            cu_seqlens=self.cu_seqlens.astype(np.int64),
            initial_state=None if self.initial_state is None
            else self.initial_state.astype(np.float64),
        )


def make_inputs(
    seqlens: Sequence[int],
    hk: int,
    hv: int,
    dk: int,
    dv: int,
    *,
    seed: int,
    io_dtype: str = "bf16",
    gate_dtype: str = "f32",
    init_state: bool = False,
    state_std: float = 0.02,
) -> GdnInputs:
    """Draw one packed batch. Draw order: q, k, v, g, beta, initial state."""
    if hv % hk != 0:
        raise ValueError("hv must be a multiple of hk")
    seqlens = [int(s) for s in seqlens]
    if any(s < 0 for s in seqlens):
        raise ValueError("negative sequence length")
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    q = _unit_rows(rng, (T, hk, dk))
    k = _unit_rows(rng, (T, hk, dk))
    v = rng.standard_normal(size=(T, hv, dv))
    g = _neg_softplus(rng.normal(-1.0, 1.0, size=(T, hv)))
    beta = _sigmoid(rng.standard_normal(size=(T, hv)))
    s0 = None
    if init_state:
        s0 = (rng.standard_normal(size=(len(seqlens), hv, dv, dk)) * state_std).astype(np.float32)
    return GdnInputs(
        q=to_storage(q, io_dtype), k=to_storage(k, io_dtype), v=to_storage(v, io_dtype),
        g=to_storage(g, gate_dtype), beta=to_storage(beta, gate_dtype),
        cu_seqlens=cu, initial_state=s0, hk=hk, hv=hv, dk=dk, dv=dv,
        io_dtype=io_dtype, gate_dtype=gate_dtype,
    )


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> list:
    """n sequence lengths, uniform integers in [lo, hi], from their own stream."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def decode_state(batch: int, hv: int, dv: int, dk: int, *, seed: int, std: float = 0.02) -> np.ndarray:
    """Resident fp32 states [batch, HV, dv, dk] ~ N(0, std**2)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(size=(batch, hv, dv, dk)) * std).astype(np.float32)


def norm_weight(dv: int, *, seed: int) -> np.ndarray:
    """Synthetic output-normalisation weights, fp32 [dv] ~ U(0.5, 1.5)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, size=dv).astype(np.float32)


# --------------------------------------------------------------------------
# The named workloads
# --------------------------------------------------------------------------

QWEN_HEADS = dict(hk=16, hv=32, dk=128, dv=128)


def workload(name: str, io_dtype: Optional[str] = None, **overrides) -> GdnInputs:
    """Synthetic inputs for a named workload.

    tiny        1 sequence, T=64, 2 heads, d=16, fp32 (chunk 16 when prefilled)
    decode      one token for each of `batch` sequences (default 64), HK=16,
                HV=32, d=128, bf16 q/k/v and gates; states come from decode_state
    prefill     1 sequence, T=4096, HK=16, HV=32, d=128, bf16 q/k/v, fp32 gates,
                zero initial state
    long        1 sequence, T=32768, as prefill, initial state ~ N(0, 0.02^2)
    varlen      8 sequences, lengths uniform in [256, 16384], per-sequence
                initial states
    """
    if name == "tiny":
        kw = dict(seqlens=[64], hk=2, hv=2, dk=16, dv=16, seed=SEED_BASE + 0,
                  io_dtype=io_dtype or "f32", gate_dtype="f32", init_state=False)
    elif name == "decode":
        batch = overrides.pop("batch", 64)
        kw = dict(seqlens=[1] * batch, seed=SEED_BASE + 1, io_dtype=io_dtype or "bf16",
                  gate_dtype="bf16" if (io_dtype or "bf16") == "bf16" else "f32",
                  init_state=False, **QWEN_HEADS)
    elif name == "prefill":
        kw = dict(seqlens=[4096], seed=SEED_BASE + 2, io_dtype=io_dtype or "bf16",
                  gate_dtype="f32", init_state=False, **QWEN_HEADS)
    elif name == "long":
        kw = dict(seqlens=[32768], seed=SEED_BASE + 3, io_dtype=io_dtype or "bf16",
                  gate_dtype="f32", init_state=True, **QWEN_HEADS)
    elif name == "varlen":
        lens = varlen_lengths(8, 256, 16384, seed=SEED_BASE + 4 + 1000)
        kw = dict(seqlens=lens, seed=SEED_BASE + 4, io_dtype=io_dtype or "bf16",
                  gate_dtype="f32", init_state=True, **QWEN_HEADS)
    else:
        raise ValueError(f"unknown workload {name!r}")
    kw.update(overrides)
    return make_inputs(**kw)
