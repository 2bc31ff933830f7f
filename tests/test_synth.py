"""The seeded input generator: determinism, storage rounding, distributions."""

import os

import numpy as np
import pytest
import torch

import gdn_synth as gs


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check_rne(u32: np.ndarray):
    x = u32.view(np.float32)
    mine = gs.f32_to_bf16_bits(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    # NaN stays NaN
    assert np.all(np.isnan(gs.bf16_bits_to_f32(mine[nan])))


def test_bf16_rne_every_high_half_every_rounding_class():
    """All 65536 sign/exponent/mantissa prefixes, each with every class of low
    half that rounding can see: zero, just above zero, just below the tie, the
    tie, just above the tie, the maximum, and random values."""
    rng = np.random.default_rng(0)
    lows = np.concatenate([
        np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32),
        rng.integers(0, 1 << 16, size=24, dtype=np.uint32)])
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    _check_rne(u)


def _rne_slice(c: int, n: int = 1 << 24) -> int:
    """Mismatches of the generator's rounding against torch's (nearest, ties
    to even) over the float32 bit patterns [c n, (c + 1) n); every NaN must
    stay a NaN."""
    u = np.arange(c * n, (c + 1) * n, dtype=np.uint64).astype(np.uint32) if (c + 1) * n > 0xFFFFFFFF \
        else np.arange(c * n, (c + 1) * n, dtype=np.uint32)
    x = u.view(np.float32)
    mine = gs.f32_to_bf16_bits(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    bad = int(np.count_nonzero((mine != ref) & ~nan))
    if nan.any():
        bad += int(np.count_nonzero(~np.isnan(gs.bf16_bits_to_f32(mine[nan]))))
    return bad


def test_bf16_rne_exhaustive():
    """Every one of the 2^32 float32 bit patterns, as the third page checks
    its conversions over all float32 values ("On descend d'un cran : #004 le
    meme compilateur sur les puces d'Apple", section "Le f16"). About 12 s on
    8 threads."""
    import concurrent.futures as cf
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        bad = sum(ex.map(_rne_slice, range(256)))
    assert bad == 0


def test_bf16_widen_is_exact():
    b = np.arange(1 << 16, dtype=np.uint16)
    f = gs.bf16_bits_to_f32(b)
    back = gs.f32_to_bf16_bits(f)
    fin = ~np.isnan(f)
    assert np.array_equal(back[fin], b[fin])


def test_deterministic_per_seed():
    a = gs.workload("tiny")
    b = gs.workload("tiny")
    for f in ("q", "k", "v", "g", "beta", "cu_seqlens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = gs.make_inputs([64], 2, 2, 16, 16, seed=gs.SEED_BASE + 99, io_dtype="f32")
    assert not np.array_equal(a.q, c.q)


def test_distributions_and_shapes():
    inp = gs.make_inputs([300, 212], 4, 8, 32, 32, seed=5, io_dtype="bf16",
                         gate_dtype="f32", init_state=True)
    w = inp.widened()
    assert w["q"].shape == (512, 4, 32) and w["v"].shape == (512, 8, 32)
    assert w["g"].shape == (512, 8) and inp.initial_state.shape == (2, 8, 32, 32)
    assert list(inp.cu_seqlens) == [0, 300, 512]
    # unit rows up to bf16 rounding
    nq = np.linalg.norm(w["q"], axis=-1)
    assert np.all(np.abs(nq - 1) < 1e-2)
    # gates: g <= 0 (a in (0, 1]); b in (0, 1)
    assert np.all(w["g"] <= 0) and np.all((w["beta"] > 0) & (w["beta"] < 1))
    # E[log a] = -E[softplus(N(-1,1))] ~ -0.41
    assert abs(w["g"].mean() + 0.41) < 0.05
    assert abs(inp.initial_state.std() - 0.02) < 0.002


def test_named_workloads_shapes():
    t = gs.workload("tiny")
    assert t.io_dtype == "f32" and t.q.shape == (64, 2, 16) and t.q.dtype == np.float32
    d = gs.workload("decode", batch=3)
    assert d.q.shape == (3, 16, 128) and d.q.dtype == np.uint16 and d.g.dtype == np.uint16
    lens = gs.varlen_lengths(8, 256, 16384, seed=gs.SEED_BASE + 4 + 1000)
    assert len(lens) == 8 and all(256 <= x <= 16384 for x in lens)
