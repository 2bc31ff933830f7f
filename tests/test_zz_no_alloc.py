"""gdn_prefill_noalloc (the library's fixed device workspace) against
gdn_prefill with a caller workspace: two calls in a row, the second smaller,
each bit-identical to the ordinary entry point and within the oracle's bar."""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import device_inputs, note, oracle_ref, rel_err, requires_gpu, to_f64, tol

pytestmark = [pytest.mark.gpu, requires_gpu]


def _both(inp, chunk):
    d = device_inputs(inp)
    T, N = inp.total_tokens, inp.num_seqs
    odt = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    out_a = torch.full((T, inp.hv, inp.dv), float("nan"), dtype=odt, device="cuda")
    fin_a = torch.full((N, inp.hv, inp.dv, inp.dk), float("nan"), dtype=torch.float32, device="cuda")
    note(f"prefill_noalloc lens={np.diff(inp.cu_seqlens).tolist()} chunk={chunk}")
    gdn.prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], out=out_a,
                        final_state=fin_a, initial_state=d["initial_state"], chunk=chunk)
    torch.cuda.synchronize()
    note(f"prefill (caller workspace) lens={np.diff(inp.cu_seqlens).tolist()} chunk={chunk}")
    out_b, fin_b = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                               initial_state=d["initial_state"])
    torch.cuda.synchronize()
    return out_a, fin_a, out_b, fin_b


def test_noalloc_two_calls_match_prefill():
    # 1: the prefill workload (T = 4096, HK = 16, HV = 32, d = 128, bf16)
    big = gs.workload("prefill", io_dtype="bf16")
    oa, fa, ob, fb = _both(big, 64)
    assert torch.equal(oa, ob) and torch.equal(fa, fb)
    o_ref, f_ref = oracle_ref(big)
    assert rel_err(to_f64(oa), o_ref) <= tol("bf16")
    assert rel_err(to_f64(fa), f_ref) <= tol("bf16")
    # 2: smaller, two ragged sequences with initial states, after the first
    # call has left its contents in the shared array
    small = gs.make_inputs([300, 77], 16, 32, 128, 128, seed=gs.SEED_BASE + 901, io_dtype="bf16",
                           gate_dtype="f32", init_state=True)
    oa, fa, ob, fb = _both(small, 64)
    assert torch.equal(oa, ob) and torch.equal(fa, fb)
    o_ref, f_ref = oracle_ref(small)
    assert rel_err(to_f64(oa), o_ref) <= tol("bf16")
    assert rel_err(to_f64(fa), f_ref) <= tol("bf16")


def test_noalloc_fp32_and_chunk0():
    """fp32 I/O at its 1e-4 bar, and chunk 0 (the rule's method)."""
    inp = gs.make_inputs([200, 0, 130], 2, 4, 64, 64, seed=gs.SEED_BASE + 902, io_dtype="f32",
                         gate_dtype="f32", init_state=True)
    for chunk in (32, 0):
        oa, fa, ob, fb = _both(inp, chunk)
        assert torch.equal(oa, ob) and torch.equal(fa, fb)
        o_ref, f_ref = oracle_ref(inp)
        assert rel_err(to_f64(oa), o_ref) <= tol("f32")
        assert rel_err(to_f64(fa), f_ref) <= tol("f32")


def test_noalloc_rejects_what_does_not_fit():
    """More workspace than the fixed array holds: GDN_ERR_WORKSPACE before
    anything is launched (T = 32768 at chunk 64 needs about 800 MB)."""
    T = 32768
    q = torch.zeros((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, 32), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    out = torch.empty_like(v)
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill_noalloc(q, q, v, g, g, cu, out=out, chunk=64)
    assert e.value.status == 4
