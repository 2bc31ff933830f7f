"""The chunked scan with 32, 64 or 128 state rows per workgroup.

On bf16 I/O, the scan gives each workgroup the fewest value rows of a state
(16, 32, 64 or 128, at most d) whose workgroups fit the GPU's 256 CUs in one
pass (N * HV * DV / rows <= 256), else the most. Every output and state
element goes through the same MFMA sequence whatever the rows, so a batched
call must give the same bits as calls on each sequence alone, which fit one
pass and keep 16-row slices (1 * HV * DV / 16 <= 256). Both are held to the
bf16 bar against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import TOL_BF16, device_inputs, note, oracle_ref, rel_err, requires_gpu, run_prefill, to_f64

pytestmark = [pytest.mark.gpu, requires_gpu]

CUS = 256


def _wide(n, hv, d):
    return n * hv * (d // 16) > CUS


def _batch_for(rows, hv, d):
    """The fewest sequences for which the scan takes `rows` state rows."""
    return CUS // (hv * d // (rows // 2)) + 2


def _lengths(n, seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, 150, size=n)]
    lens[1] = 0      # an empty sequence
    lens[2] = 64     # exactly one chunk of 64
    return lens


def _call(q, k, v, g, b, cu, s0, chunk, state_dtype):
    return gdn.prefill(q, k, v, g, b, cu, chunk=chunk, scale=0.8, initial_state=s0, state_dtype=state_dtype)


@pytest.mark.parametrize("d,chunk,state,rows", [(32, 16, "f32", 32), (32, 32, "f32", 32), (32, 64, "f32", 32),
                                                (64, 16, "f32", 32), (64, 32, "f32", 32), (64, 64, "f32", 32),
                                                (128, 16, "f32", 32), (128, 32, "f32", 32), (128, 64, "f32", 32),
                                                (128, 64, "bf16", 32),
                                                (64, 16, "f32", 64), (64, 64, "f32", 64), (64, 64, "bf16", 64),
                                                (128, 16, "f32", 64), (128, 32, "f32", 64), (128, 64, "f32", 64),
                                                (128, 16, "f32", 128), (128, 32, "f32", 128),
                                                (128, 64, "f32", 128), (128, 64, "bf16", 128)])
def test_wide_slices_match_single_sequence_calls(d, chunk, state, rows):
    hk, hv = 4, 8
    n = _batch_for(rows, hv, d)
    assert _wide(n, hv, d) and not _wide(1, hv, d)
    assert gdn.prefill_plan(n, n * 100, hk, hv, d, chunk) == (chunk, rows)
    lens = _lengths(n, seed=1200 + d + chunk + rows)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=1300 + d + chunk + rows, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    sd = torch.bfloat16 if state == "bf16" else torch.float32
    note(f"wide slices d={d} chunk={chunk} state={state} rows={rows} N={n}")
    t = device_inputs(inp)
    s0 = t["initial_state"] if state == "f32" else t["initial_state"].to(torch.bfloat16)
    o, f = _call(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], s0, chunk, sd)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens
    for i in range(n):
        a, e = int(cu[i]), int(cu[i + 1])
        if a == e:
            assert torch.equal(f[i], s0[i])
            continue
        one = torch.tensor([0, e - a], dtype=torch.int32, device="cuda")
        oi, fi = _call(t["q"][a:e].contiguous(), t["k"][a:e].contiguous(), t["v"][a:e].contiguous(),
                       t["g"][a:e].contiguous(), t["beta"][a:e].contiguous(), one, s0[i:i + 1].contiguous(),
                       chunk, sd)
        torch.cuda.synchronize()
        assert torch.equal(o[a:e], oi), f"sequence {i}: outputs differ from its own call"
        assert torch.equal(f[i], fi[0]), f"sequence {i}: final state differs from its own call"
    # bf16 states: the oracle starts from the rounded initial state
    o_ref, f_ref = oracle_ref(inp, scale=0.8, initial_state=None if state == "f32" else to_f64(s0))
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] wide slices d={d} chunk={chunk} state={state} rows={rows} N={n} out_err={eo:.3e} "
          f"state_err={ef:.3e}",
          flush=True)
    assert eo <= TOL_BF16 and ef <= TOL_BF16


def test_wide_slices_many_heads_one_sequence():
    """48 value heads of d = 128 (384 16-row slices): one sequence alone
    takes 32-row slices; every head against the oracle."""
    inp = gs.make_inputs([300], 16, 48, 128, 128, seed=1401, io_dtype="bf16", gate_dtype="f32", init_state=True)
    assert _wide(1, 48, 128)
    note("wide slices 48 heads")
    t = device_inputs(inp)
    o, f = gdn.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], chunk=64,
                       initial_state=t["initial_state"])
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_ref(inp)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] wide slices 48 heads out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= TOL_BF16 and ef <= TOL_BF16


@pytest.mark.parametrize("hk,hv,d,rows", [(8, 8, 128, 128), (2, 8, 128, 128), (1, 8, 128, 64), (4, 16, 64, 64),
                                          (3, 12, 128, 32)])
def test_wide_slices_head_groups(hk, hv, d, rows):
    """Value heads per query/key head of 1, 4 and 8 (the scan places a q/k
    head's slices together; the grid pads the groups), d = 64, and a q/k
    head count that is not a power of two: every head against the oracle,
    and sequences 0 and 3 bit for bit against their own calls."""
    n = _batch_for(rows, hv, d)
    assert gdn.prefill_plan(n, n * 100, hk, hv, d, 64) == (64, rows)
    lens = _lengths(n, seed=1500 + hk + hv + d + rows)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=1600 + hk + hv + d + rows, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    note(f"wide slices hk={hk} hv={hv} d={d} rows={rows} N={n}")
    t = device_inputs(inp)
    s0 = t["initial_state"]
    o, f = _call(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu_seqlens"], s0, 64, torch.float32)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens
    for i in (0, 3):
        a, e = int(cu[i]), int(cu[i + 1])
        one = torch.tensor([0, e - a], dtype=torch.int32, device="cuda")
        oi, fi = _call(t["q"][a:e].contiguous(), t["k"][a:e].contiguous(), t["v"][a:e].contiguous(),
                       t["g"][a:e].contiguous(), t["beta"][a:e].contiguous(), one, s0[i:i + 1].contiguous(),
                       64, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o[a:e], oi) and torch.equal(f[i], fi[0]), f"sequence {i} differs from its own call"
    o_ref, f_ref = oracle_ref(inp, scale=0.8)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] wide slices hk={hk} hv={hv} d={d} rows={rows} N={n} out_err={eo:.3e} state_err={ef:.3e}",
          flush=True)
    assert eo <= TOL_BF16 and ef <= TOL_BF16


def test_max_seqlen_hint_changes_rows_not_results():
    """An uneven batch (one 2,048-token prompt beside four of 256): the
    one-pass rule takes 128-row slices; with the longest length as a hint
    the rule takes 32-row slices, which finish sooner. Same chunk size, so
    outputs and final states are bit for bit those of the call without the
    hint, and both meet the oracle's bar. A hint below the mean length or
    above the total is refused."""
    lens = [2048, 256, 256, 256, 256]
    N, T = len(lens), sum(lens)
    assert gdn.prefill_plan(N, T, 16, 32, 128) == (64, 128)
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=2048) == (64, 32)
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 1700, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    note("prefill max_seqlen hint 2048 + 4 x 256")
    o0, f0 = run_prefill(inp, chunk=0)
    o1, f1 = run_prefill(inp, chunk=0, max_seqlen=2048)
    assert torch.equal(o0, o1) and torch.equal(f0, f1)
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o1), o_ref) <= TOL_BF16 and rel_err(to_f64(f1), f_ref) <= TOL_BF16
    for bad in (T // N - 1, T + 1):
        with pytest.raises(gdn.GdnError):
            run_prefill(inp, chunk=0, max_seqlen=bad)


def test_max_seqlen_hint_chunks_tiny_sequences():
    """300 tokens beside 40 single-token sequences: the mean length (8.3)
    sends the batch token by token, but the longest sequence sets the token
    scan's time; with the hint the batch is chunked (chunks of 32, 128 state
    rows). Both calls meet the oracle's bar."""
    lens = [300] + [1] * 40
    N, T = len(lens), sum(lens)
    assert gdn.prefill_plan(N, T, 16, 32, 128) == (1, 0)
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=300) == (32, 128)
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 1710, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    note("prefill max_seqlen hint 300 + 40 x 1")
    o_ref, f_ref = oracle_ref(inp)
    for hint in (None, 300):
        o, f = run_prefill(inp, chunk=0, max_seqlen=hint)
        eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
        print(f"[parity] hint={hint} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
        assert eo <= TOL_BF16 and ef <= TOL_BF16
