"""Token-by-token prefill (gdn_prefill with chunk 1, and chunk 0 on short
prompts) on the GPU against the fp64 oracle.

The same bars as the chunked path, max |gpu - ref| / max |ref| per tensor:
bf16 I/O <= 2e-2, fp32 I/O <= 1e-4. Every workload is compared over all of
its value heads and tokens.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import (TOL_F32, device_inputs, note, oracle_ref, rel_err, requires_gpu, run_prefill,
                      to_f64, tol)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _check(inp, o, f, *, heads=None, scale=1.0, label=""):
    io = inp.io_dtype
    o_ref, f_ref = oracle_ref(inp, heads=heads, scale=scale)
    og, fg = to_f64(o), to_f64(f)
    if heads is not None:
        og, o_ref = og[:, heads], o_ref[:, heads]
        fg, f_ref = fg[:, heads], f_ref[:, heads]
    assert np.isfinite(og).all(), f"{label}: unwritten (NaN) outputs"
    eo, ef = rel_err(og, o_ref), rel_err(fg, f_ref)
    print(f"[parity] token-scan {label} io={io} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(io), f"{label}: output error {eo}"
    assert ef <= tol(io), f"{label}: final state error {ef}"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_token_scan_tiny(io):
    inp = gs.workload("tiny", io_dtype=io)
    note(f"token scan tiny io={io}")
    o, f = run_prefill(inp, chunk=1)
    _check(inp, o, f, label="tiny")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_token_scan_ragged(d, io):
    """Several sequences, ragged lengths, an empty one, initial states, scale;
    every head size (rows of 2 to 16 lanes)."""
    inp = gs.make_inputs([1, 70, 0, 130, 33], 2, 4, d, d, seed=51 + d, io_dtype=io, gate_dtype="f32",
                         init_state=True)
    note(f"token scan ragged d={d} io={io}")
    o, f = run_prefill(inp, chunk=1, scale=0.75)
    _check(inp, o, f, scale=0.75, label=f"ragged d={d}")
    assert np.array_equal(to_f64(f)[2], inp.initial_state[2].astype(np.float64))


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_token_scan_multi_token_steps(d, io):
    """Sequences of 1 to 4 tokens take a direct path (one per length), 5 and
    more the pipelined one; with initial states, as in a multi-token step."""
    lens = [1, 2, 3, 4, 5, 0, 4, 1, 9]
    inp = gs.make_inputs(lens, 2, 4, d, d, seed=71 + d, io_dtype=io, gate_dtype=io, init_state=True)
    note(f"token scan multi-token steps d={d} io={io}")
    o, f = run_prefill(inp, chunk=1, scale=0.5)
    _check(inp, o, f, scale=0.5, label=f"steps d={d}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_token_scan_prefill_4k(io):
    """The prefill workload (T = 4096, HK = 16, HV = 32, d = 128) token by
    token: one sequence, bf16 gates as loaded."""
    inp = gs.workload("prefill", io_dtype=io)
    note(f"token scan T=4096 io={io}")
    o, f = run_prefill(inp, chunk=1)
    _check(inp, o, f, label="T=4096")


def test_token_scan_varlen_f32():
    """8 packed sequences of 256 .. 16384 tokens with their own initial states."""
    inp = gs.workload("varlen", io_dtype="f32")
    note(f"token scan varlen lens={np.diff(inp.cu_seqlens).tolist()}")
    o, f = run_prefill(inp, chunk=1)
    _check(inp, o, f, label="varlen")


def test_token_scan_equals_chunked_fp32():
    """Both evaluations of one recurrence agree to fp32 rounding."""
    inp = gs.make_inputs([300, 1, 77], 2, 4, 64, 64, seed=61, io_dtype="f32", gate_dtype="f32",
                         init_state=True)
    note("token scan vs chunked")
    o1, f1 = run_prefill(inp, chunk=1)
    o64, f64 = run_prefill(inp, chunk=64)
    assert rel_err(to_f64(o1), to_f64(o64)) <= TOL_F32
    assert rel_err(to_f64(f1), to_f64(f64)) <= TOL_F32


def test_token_scan_in_place_and_empty():
    """final_state may be initial_state; with every sequence empty (T = 0)
    the states pass through and nothing is read."""
    inp = gs.make_inputs([40, 9], 2, 4, 32, 32, seed=63, io_dtype="f32", gate_dtype="f32",
                         init_state=True)
    d = device_inputs(inp)
    s = d["initial_state"].clone()
    note("token scan in place")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=1,
                       initial_state=s, final_state=s)
    torch.cuda.synchronize()
    assert f.data_ptr() == s.data_ptr()
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o), o_ref) <= TOL_F32 and rel_err(to_f64(f), f_ref) <= TOL_F32
    empty = gs.make_inputs([0, 0], 2, 4, 32, 32, seed=64, io_dtype="bf16", init_state=True)
    note("token scan with every sequence empty")
    o, f = run_prefill(empty, chunk=1)
    assert o.shape[0] == 0 and np.array_equal(to_f64(f), empty.initial_state.astype(np.float64))


def test_token_scan_malformed_cu_seqlens_is_clamped():
    """Same clamping of cu_seqlens as the chunked path: no fault, and the
    well-formed sequence before the bad offsets is right."""
    inp = gs.make_inputs([50, 30], 2, 2, 32, 32, seed=21, io_dtype="f32")
    d = device_inputs(inp)
    cu_bad = torch.tensor([0, 50, 10, 9999], dtype=torch.int32, device="cuda")
    note("token scan malformed cu_seqlens")
    out1 = torch.zeros((80, 2, 32), dtype=torch.float32, device="cuda")
    out16 = torch.zeros((80, 2, 32), dtype=torch.float32, device="cuda")
    o1, f1 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_bad, chunk=1, out=out1)
    o16, f16 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_bad, chunk=16, out=out16)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o1)[:50], o_ref[:50]) <= TOL_F32
    assert rel_err(to_f64(f1)[0], f_ref[0]) <= TOL_F32
    # both paths read the same clamped bounds
    assert rel_err(to_f64(o1), to_f64(o16)) <= TOL_F32
    assert rel_err(to_f64(f1), to_f64(f16)) <= TOL_F32


@pytest.mark.parametrize("lens,expect", [([30], "token_scan"), ([48], "scan"), ([100], "scan"),
                                         ([10] * 16, "token_scan"), ([12] * 16, "scan"), ([30] * 16, "scan")])
def test_chunk_zero_picks_by_length(lens, expect):
    """chunk 0 with nothing tuned: token by token when T <= 32 or the mean
    length is at most 10 tokens, chunked above (the method the library
    reports for the sizes is the one that runs)."""
    inp = gs.make_inputs(lens, 2, 4, 32, 32, seed=65, io_dtype="bf16", gate_dtype="f32")
    d = device_inputs(inp)
    note(f"chunk 0 with lengths {lens}")
    gdn.timing_start(8)
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=0)
    kt = gdn.timing_stop()
    torch.cuda.synchronize()
    ran = {k for k, v in kt.items() if v.get("count", 0)}
    assert expect in ran, ran
    assert ("token_scan" in ran) != ("scan" in ran), ran
    m = gdn.prefill_method(len(lens), sum(lens), 2, 4, 32)
    assert (m == 1) == (expect == "token_scan"), m
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o), o_ref) <= tol("bf16") and rel_err(to_f64(f), f_ref) <= tol("bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_token_scan_paired_rows_on_batches(d, io):
    """64 sequences x 32 value heads is enough workgroups for the kernel to
    hold two state rows per lane group: ragged lengths (empty, 1-4 tokens on
    the direct path, 5-70 through the block ring), initial states, every
    head compared."""
    rng = np.random.default_rng(90 + d)
    lens = [int(x) for x in rng.choice([0, 1, 2, 3, 4, 5, 9, 17, 64, 70], size=64)]
    inp = gs.make_inputs(lens, 16, 32, d, d, seed=91 + d, io_dtype=io, gate_dtype=io, init_state=True)
    note(f"token scan paired rows d={d} io={io}")
    o, f = run_prefill(inp, chunk=1, scale=0.5)
    _check(inp, o, f, scale=0.5, label=f"paired d={d}")
