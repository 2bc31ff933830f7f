"""Chunked prefill on the GPU against the fp64 oracle.

Workloads (gdn_synth.workload): tiny (T=64, d=16, fp32), prefill (T=4096,
HK=16, HV=32, d=128), long (T=32768, nonzero initial state), varlen (8
sequences, lengths in [256, 16384], per-sequence initial states, then 64
decode steps). Bars, as max |gpu - ref| / max |ref| per tensor:
  bf16 I/O: outputs <= 2e-2, final states <= 2e-2 (bf16 MFMA operands);
  fp32 I/O: outputs and final states <= 1e-4.
Every workload is compared over all of its value heads and tokens.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle
from gpu_util import (TOL_BF16, TOL_F32, device_inputs, note, oracle_ref, rel_err, requires_gpu,
                      run_prefill, to_f64, tol)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _check_ref(o, f, o_ref, f_ref, *, io, label=""):
    og, fg = to_f64(o), to_f64(f)
    assert np.isfinite(og).all(), f"{label}: unwritten (NaN) outputs"
    eo, ef = rel_err(og, o_ref), rel_err(fg, f_ref)
    print(f"[parity] {label} io={io} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(io), f"{label}: output error {eo}"
    assert ef <= tol(io), f"{label}: final state error {ef}"
    return eo, ef


def _check(inp, o, f, *, heads=None, scale=1.0, io=None, label=""):
    io = io or inp.io_dtype
    o_ref, f_ref = oracle_ref(inp, heads=heads, scale=scale)
    og, fg = to_f64(o), to_f64(f)
    if heads is not None:
        og, o_ref = og[:, heads], o_ref[:, heads]
        fg, f_ref = fg[:, heads], f_ref[:, heads]
    assert np.isfinite(og).all(), f"{label}: unwritten (NaN) outputs"
    eo, ef = rel_err(og, o_ref), rel_err(fg, f_ref)
    print(f"[parity] {label} io={io} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(io), f"{label}: output error {eo}"
    assert ef <= tol(io), f"{label}: final state error {ef}"
    return eo, ef


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_tiny(io, chunk):
    inp = gs.workload("tiny", io_dtype=io)
    note(f"prefill tiny io={io} chunk={chunk}")
    o, f = run_prefill(inp, chunk=chunk)
    _check(inp, o, f, label=f"tiny C={chunk}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_ragged_varlen_small(d, chunk):
    """Several sequences, ragged tails, an empty sequence, initial states, scale."""
    inp = gs.make_inputs([1, 70, 0, 130, 33], 2, 4, d, d, seed=31 + d, io_dtype="f32",
                         gate_dtype="f32", init_state=True)
    note(f"prefill ragged d={d} chunk={chunk}")
    o, f = run_prefill(inp, chunk=chunk, scale=0.75)
    _check(inp, o, f, scale=0.75, label=f"ragged d={d} C={chunk}")
    # the empty sequence passes its initial state through unchanged
    assert np.array_equal(to_f64(f)[2], inp.initial_state[2].astype(np.float64))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prefill_4k(io):
    inp = gs.workload("prefill", io_dtype=io)
    note(f"prefill T=4096 io={io}")
    o, f = run_prefill(inp, chunk=64)
    _check(inp, o, f, label="prefill T=4096")


def _segment_errors(o, o_ref, heads, seg=4096):
    """max |gpu - ref| per segment of `seg` tokens, over the given heads,
    relative to the largest reference magnitude of the whole sequence."""
    og, orf = to_f64(o)[:, heads], o_ref[:, heads]
    den = float(np.abs(orf).max())
    return [float(np.abs(og[t:t + seg] - orf[t:t + seg]).max()) / den for t in range(0, len(orf), seg)]


ALL_HEADS = list(range(32))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_long_32k(io):
    """T = 32768 with an initial state, every value head; the error is also
    reported per 4096-token segment, to show whether it grows along the state
    carry."""
    inp = gs.workload("long", io_dtype=io)
    note(f"prefill T=32768 io={io}")
    o, f = run_prefill(inp, chunk=64)
    o_ref, f_ref = oracle_ref(inp)
    _check_ref(o, f, o_ref, f_ref, io=io, label="long T=32768")
    errs = _segment_errors(o, o_ref, ALL_HEADS)
    print(f"[segments] long T=32768 io={io} out_err per 4K: " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= tol(io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_long_no_decay_stress(io):
    """a = 1 everywhere: the state carries over all 32768 tokens (it stays
    bounded because I - b k k^T is a contraction). Every value head, against
    the oracle; in fp32 I/O the error must not grow along the carry."""
    inp = gs.workload("long", io_dtype=io)
    inp.g[:] = 0.0
    note(f"prefill T=32768 g=0 stress io={io}")
    o, f = run_prefill(inp, chunk=64)
    o_ref, f_ref = oracle_ref(inp)
    _check_ref(o, f, o_ref, f_ref, io=io, label="long g=0")
    errs = _segment_errors(o, o_ref, ALL_HEADS)
    print(f"[segments] long g=0 {io} out_err per 4K: " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    if io == "f32":
        # carried over all 32768 tokens, the error must not grow: the last
        # segment stays within a few times the first
        assert errs[-1] <= 4 * errs[0] + 1e-6


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_varlen_then_decode(io):
    """8 packed sequences with their own initial states, then 64 decode steps
    continuing every sequence from its final prefill state."""
    inp = gs.workload("varlen", io_dtype=io)
    note(f"prefill varlen io={io} lens={np.diff(inp.cu_seqlens).tolist()}")
    o, f = run_prefill(inp, chunk=64)
    o_pre, f_ref = oracle_ref(inp)
    _check_ref(o, f, o_pre, f_ref, io=io, label="varlen")
    del o_pre
    # continue with 64 decode steps from the GPU's own final states
    N = inp.num_seqs
    state = f.clone()
    dec = gs.make_inputs([64] * N, 16, 32, 128, 128, seed=gs.SEED_BASE + 404, io_dtype=io,
                         gate_dtype=io)
    w = dec.widened()
    # the reference continues from the oracle's prefill state
    dd = device_inputs(dec)
    outs = []
    for t in range(64):
        idx = torch.arange(N, device="cuda") * 64 + t
        out = gdn.decode_step(dd["q"][idx].contiguous(), dd["k"][idx].contiguous(),
                              dd["v"][idx].contiguous(), dd["g"][idx].contiguous(),
                              dd["beta"][idx].contiguous(), state)
        outs.append(out)
    torch.cuda.synchronize()
    got = np.stack([to_f64(x) for x in outs], axis=1)  # [N, 64, hv, dv]
    o_ref, s_ref = oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"],
                               initial_state=f_ref)
    o_ref = o_ref.reshape(N, 64, 32, 128)
    e_o = rel_err(got, o_ref)
    e_s = rel_err(to_f64(state), s_ref)
    print(f"[parity] varlen+64 decode io={io} out_err={e_o:.3e} state_err={e_s:.3e}", flush=True)
    assert e_o <= tol(io) and e_s <= tol(io)


# ------------------------------------------------------------------ invariants

def test_no_write_no_decay_is_identity():
    """b = 0, g = 0: the final state equals the initial state and
    o_t = scale S0 q_t."""
    inp = gs.make_inputs([100], 2, 4, 64, 64, seed=5, io_dtype="f32", init_state=True)
    inp.beta[:] = 0.0
    inp.g[:] = 0.0
    note("prefill identity")
    o, f = run_prefill(inp, chunk=32, scale=2.0)
    assert rel_err(to_f64(f), inp.initial_state.astype(np.float64)) <= 1e-6
    w = inp.widened()
    for h in range(4):
        ref = 2.0 * w["q"][:, h // 2] @ w["initial_state"][0, h].T
        assert rel_err(to_f64(o)[:, h], ref) <= TOL_F32


def test_retrieval_standard_basis_bf16():
    """a = 1, b = 1, distinct standard-basis keys within each head, zero state:
    querying key e_j returns the value stored there."""
    T, hk, hv, d = 64, 2, 4, 128
    q = np.zeros((T, hk, d))
    k = np.zeros((T, hk, d))
    for t in range(T):
        for kh in range(hk):
            k[t, kh, (t * 2 + kh) % d] = 1.0
            q[t, kh, (t * 2 + kh) % d] = 1.0
    rng = np.random.default_rng(1)
    v = rng.standard_normal((T, hv, d))
    inp = gs.GdnInputs(q=gs.to_storage(q, "bf16"), k=gs.to_storage(k, "bf16"),
                       v=gs.to_storage(v, "bf16"), g=np.zeros((T, hv), np.float32),
                       beta=np.ones((T, hv), np.float32), cu_seqlens=np.array([0, T], np.int32),
                       initial_state=None, hk=hk, hv=hv, dk=d, dv=d, io_dtype="bf16",
                       gate_dtype="f32")
    note("prefill retrieval")
    o, f = run_prefill(inp, chunk=64)
    vb = gs.widen(inp.v, "bf16")
    np.testing.assert_array_equal(to_f64(o), vb)
    # and the final state maps every key to its value
    fs = to_f64(f)[0]
    for t in range(T):
        for h in range(hv):
            np.testing.assert_allclose(fs[h] @ k[t, h // 2], vb[t, h], rtol=0, atol=1e-2)


def test_split_prefill_equals_one_call():
    inp = gs.make_inputs([300], 2, 4, 128, 128, seed=8, io_dtype="f32", init_state=True)
    note("prefill split")
    o, f = run_prefill(inp, chunk=64)
    d = device_inputs(inp)
    m = 137
    sl = lambda x, a, b: x[a:b].contiguous()
    cu1 = torch.tensor([0, m], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 300 - m], dtype=torch.int32, device="cuda")
    oa, fa = gdn.prefill(sl(d["q"], 0, m), sl(d["k"], 0, m), sl(d["v"], 0, m), sl(d["g"], 0, m),
                         sl(d["beta"], 0, m), cu1, chunk=64, initial_state=d["initial_state"])
    ob, fb = gdn.prefill(sl(d["q"], m, 300), sl(d["k"], m, 300), sl(d["v"], m, 300),
                         sl(d["g"], m, 300), sl(d["beta"], m, 300), cu2, chunk=64, initial_state=fa)
    torch.cuda.synchronize()
    assert rel_err(np.concatenate([to_f64(oa), to_f64(ob)]), to_f64(o)) <= TOL_F32
    assert rel_err(to_f64(fb), to_f64(f)) <= TOL_F32


def test_single_token_prefill_equals_decode():
    inp = gs.make_inputs([1] * 3, 16, 32, 128, 128, seed=12, io_dtype="bf16", gate_dtype="bf16",
                         init_state=True)
    note("prefill T=1 vs decode")
    o, f = run_prefill(inp, chunk=64)
    d = device_inputs(inp)
    st = d["initial_state"].clone()
    od = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st)
    torch.cuda.synchronize()
    assert rel_err(to_f64(od), to_f64(o)) <= TOL_BF16
    assert rel_err(to_f64(st), to_f64(f)) <= TOL_BF16


def test_varlen_equals_separate_calls():
    lens = [190, 64, 1, 77]
    inp = gs.make_inputs(lens, 2, 4, 64, 64, seed=13, io_dtype="bf16", init_state=True)
    note("prefill varlen vs separate")
    o, f = run_prefill(inp, chunk=32)
    d = device_inputs(inp)
    cu = inp.cu_seqlens
    for n, L in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        on, fn = gdn.prefill(*(d[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")),
                             torch.tensor([0, L], dtype=torch.int32, device="cuda"), chunk=32,
                             initial_state=d["initial_state"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(on.view(torch.int16), o[a:b].view(torch.int16))
        assert torch.equal(fn[0], f[n])


def test_deterministic_and_in_place_state():
    inp = gs.workload("prefill", io_dtype="bf16")
    note("prefill determinism")
    d = device_inputs(inp)
    o1, f1 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64)
    o2, f2 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1, f2)
    # in place: final state written over the initial state
    s = f1.clone()
    o3, f3 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                         initial_state=f1, final_state=f1)
    o4, f4 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                         initial_state=s)
    torch.cuda.synchronize()
    assert f3.data_ptr() == f1.data_ptr()
    assert torch.equal(f3, f4) and torch.equal(o3.view(torch.int16), o4.view(torch.int16))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n_seqs", [256, 300])
def test_many_short_sequences(n_seqs, io):
    """Many ragged sequences, some empty, with initial states. Up to 256 the
    preparation kernel locates its chunks itself; past that a separate
    schedule kernel builds the chunk table. Both must agree with the oracle."""
    lens = gs.varlen_lengths(n_seqs, 0, 40, seed=gs.SEED_BASE + 77)
    inp = gs.make_inputs(lens, 2, 4, 32, 32, seed=gs.SEED_BASE + 78, io_dtype=io, gate_dtype="f32",
                         init_state=True)
    note(f"prefill many sequences N={n_seqs} io={io}")
    o, f = run_prefill(inp, chunk=16)
    _check(inp, o, f, label=f"N={n_seqs}")
    empty = [i for i, n in enumerate(lens) if n == 0]
    assert empty, "the draw should include empty sequences"
    for i in empty:
        assert np.array_equal(to_f64(f)[i], inp.initial_state[i].astype(np.float64))


def test_malformed_cu_seqlens_is_clamped():
    """Offsets past the end or decreasing are clamped on the device: no fault,
    and well-formed sequences before them are still right."""
    inp = gs.make_inputs([50, 30], 2, 2, 32, 32, seed=21, io_dtype="f32")
    d = device_inputs(inp)
    cu_bad = torch.tensor([0, 50, 10, 9999], dtype=torch.int32, device="cuda")
    note("prefill malformed cu_seqlens")
    out = torch.zeros((80, 2, 32), dtype=torch.float32, device="cuda")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_bad, chunk=16, out=out)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o)[:50], o_ref[:50]) <= TOL_F32
    assert rel_err(to_f64(f)[0], f_ref[0]) <= TOL_F32


def test_all_sequences_empty():
    """T = 0: every sequence is empty, so no chunk exists. The preparation
    kernel must not read q or k (there are none), and each final state is its
    initial state."""
    inp = gs.make_inputs([0, 0, 0], 2, 4, 32, 32, seed=41, io_dtype="bf16", init_state=True)
    note("prefill with every sequence empty")
    o, f = run_prefill(inp, chunk=64)
    assert o.shape[0] == 0
    assert np.array_equal(to_f64(f), inp.initial_state.astype(np.float64))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_first_sequence_not_at_token_zero(io):
    """cu_seqlens[0] > 0: the packed buffer holds tokens before the first
    sequence. No chunk then starts at chunk_index * C, so the preparation
    kernel's early loads (made for that common layout) are all discarded and
    reloaded; results must match the oracle on the sequences proper."""
    inp = gs.make_inputs([5, 70, 33], 2, 4, 32, 32, seed=43, io_dtype=io, gate_dtype="f32",
                         init_state=True)
    d = device_inputs(inp)
    cu = d["cu_seqlens"][1:].contiguous()  # sequences 1 and 2 only; tokens 0..4 are not in any
    note(f"prefill with cu_seqlens[0] = 5 io={io}")
    out_dtype = torch.bfloat16 if io == "bf16" else torch.float32
    out = torch.full((inp.total_tokens, 4, 32), float("nan"), dtype=out_dtype, device="cuda")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, chunk=16,
                       initial_state=d["initial_state"][1:].contiguous(), out=out)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_ref(inp)
    eo = rel_err(to_f64(o)[5:], o_ref[5:])
    ef = rel_err(to_f64(f), f_ref[1:])
    print(f"[parity] cu0=5 io={io} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(io) and ef <= tol(io)
    assert torch.isnan(o[:5].float()).all(), "tokens before the first sequence must not be written"


def test_tiny_as_64_decode_steps():
    """The tiny workload (T = 64, HK = HV = 2, d = 16, fp32) run as 64
    decode steps, one token each, equals the chunked prefill (C = 16) and
    the oracle: the two GPU paths evaluate one recurrence."""
    inp = gs.workload("tiny", io_dtype="f32")
    note("tiny as 64 decode steps")
    o_p, f_p = run_prefill(inp, chunk=16)
    d = device_inputs(inp)
    state = torch.zeros((1, 2, 16, 16), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(64):
        sl = slice(t, t + 1)
        outs.append(gdn.decode_step(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], d["beta"][sl], state))
    torch.cuda.synchronize()
    o_d = torch.cat(outs, 0)
    o_ref, f_ref = oracle_ref(inp)
    e_do, e_ds = rel_err(to_f64(o_d), o_ref), rel_err(to_f64(state), f_ref)
    e_pd = rel_err(to_f64(o_d), to_f64(o_p))
    print(f"[parity] tiny as 64 decode steps out_err={e_do:.3e} state_err={e_ds:.3e} vs prefill {e_pd:.3e}",
          flush=True)
    assert e_do <= TOL_F32 and e_ds <= TOL_F32 and e_pd <= TOL_F32
    assert rel_err(to_f64(state), to_f64(f_p)) <= TOL_F32


@pytest.mark.parametrize("chunk", [64, 1])
def test_sequences_beyond_the_ranked_count(chunk):
    """4,500 sequences of 0 to 3 tokens: past 4,096 sequences the schedule
    keeps them in index order instead of longest first; results are the
    same."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(0, 4, 4500)]
    inp = gs.make_inputs(lens, 1, 2, 32, 32, seed=79, io_dtype="f32", gate_dtype="f32", init_state=True)
    note(f"prefill with {len(lens)} sequences chunk={chunk}")
    o, f = run_prefill(inp, chunk=chunk)
    o_ref, f_ref = oracle_ref(inp)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] N=4500 chunk={chunk} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= TOL_F32 and ef <= TOL_F32


@pytest.mark.parametrize("chunk", [64, 16, 1])
def test_decay_underflow_resets_the_state(chunk):
    """g = -1e4 makes a = exp(g) exactly 0: the state restarts from
    b v k^T at those tokens (every token, or a random fifth of them). The
    chunked form then holds cumulative log-decays near -6e5 and decay
    factors of exactly 0 or 1; nothing may overflow or turn NaN."""
    for frac in (1.0, 0.2):
        inp = gs.make_inputs([150, 64, 9], 2, 4, 64, 64, seed=81, io_dtype="f32", gate_dtype="f32",
                             init_state=True)
        mask = np.random.default_rng(83).random(inp.g.shape) < frac
        inp.g[mask] = np.float32(-1e4)
        note(f"decay underflow frac={frac} chunk={chunk}")
        o, f = run_prefill(inp, chunk=chunk)
        o_ref, f_ref = oracle_ref(inp)
        assert np.isfinite(to_f64(o)).all() and np.isfinite(to_f64(f)).all()
        eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
        print(f"[parity] reset frac={frac} chunk={chunk} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
        assert eo <= TOL_F32 and ef <= TOL_F32
