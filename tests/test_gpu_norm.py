"""Output normalisation on the GPU against the fp64 oracle.

gdn_decode_step_norm and gdn_prefill_norm are compared with oracle.decode_step
or oracle.scan followed by oracle.rms_norm (per (token, value head) row:
y = o w / sqrt(mean(o^2) + eps)), with synthetic weights from gdn_synth. The
bars are those of the plain calls, max |gpu - ref| / max |ref| per tensor:
bf16 I/O <= 2e-2, fp32 I/O <= 1e-4. The states must be those of the plain
calls: bit for bit in decode (shared arithmetic), and the same kernels in
prefill.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle
from gpu_util import TOL_F32, device_inputs, note, oracle_ref, rel_err, requires_gpu, to_f64, tol

pytestmark = [pytest.mark.gpu, requires_gpu]


def _weight(dv, seed=5):
    return gs.norm_weight(dv, seed=gs.SEED_BASE + 500 + seed)


def _decode_case(batch, io, *, d=128, hk=16, hv=32, seed_off=0):
    inp = gs.make_inputs([1] * batch, hk, hv, d, d, seed=gs.SEED_BASE + 1 + seed_off,
                         io_dtype=io, gate_dtype=io)
    s0 = gs.decode_state(batch, hv, d, d, seed=gs.SEED_BASE + 101 + seed_off)
    return inp, s0


@pytest.mark.parametrize("eps", [1e-6, 0.05])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [1, 64])
def test_decode_norm_matches_oracle(batch, io, eps):
    """The decode workload (HK = 16, HV = 32, d = 128, up to 64 sequences)."""
    inp, s0 = _decode_case(batch, io)
    w = _weight(128)
    note(f"decode norm batch={batch} io={io} eps={eps}")
    d = device_inputs(inp)
    state = torch.from_numpy(s0).cuda()
    plain_state = torch.from_numpy(s0).cuda()
    out = torch.full((batch, 32, 128), float("nan"), dtype=d["q"].dtype, device="cuda")
    gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=out,
                    norm_weight=torch.from_numpy(w).cuda(), norm_eps=eps)
    gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], plain_state)
    torch.cuda.synchronize()
    wd = inp.widened()
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], s0.astype(np.float64))
    y_ref = oracle.rms_norm(o_ref, w, eps)
    y = to_f64(out)
    err = rel_err(y, y_ref)
    print(f"[parity] decode norm B={batch} io={io} eps={eps} out_err={err:.3e}", flush=True)
    assert np.isfinite(y).all()
    assert err <= tol(io)
    assert rel_err(to_f64(state), s_ref) <= TOL_F32
    assert torch.equal(state, plain_state), "the fused kernel must leave the plain kernel's state bits"


@pytest.mark.parametrize("d", [16, 32, 64])
def test_decode_norm_other_head_sizes(d):
    inp, s0 = _decode_case(5, "f32", d=d, hk=2, hv=4, seed_off=3)
    w = _weight(d, seed=d)
    note(f"decode norm d={d}")
    dd = device_inputs(inp)
    state = torch.from_numpy(s0).cuda()
    out = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state, scale=0.5,
                          norm_weight=torch.from_numpy(w).cuda(), norm_eps=0.01)
    torch.cuda.synchronize()
    wd = inp.widened()
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"],
                                      s0.astype(np.float64), scale=0.5)
    assert rel_err(to_f64(out), oracle.rms_norm(o_ref, w, 0.01)) <= TOL_F32
    assert rel_err(to_f64(state), s_ref) <= TOL_F32


def test_decode_norm_state_slots_and_zero_rows():
    """Slot -1: output row of zeros, state untouched. A sequence whose output
    is exactly zero (zero state, b = 0) normalises to zeros, not NaN."""
    batch, slots_n = 6, 10
    inp, _ = _decode_case(batch, "bf16", seed_off=5)
    inp.beta[1] = gs.to_storage(np.zeros(inp.hv), "bf16")  # sequence 1 writes nothing
    pool = gs.decode_state(slots_n, 32, 128, 128, seed=gs.SEED_BASE + 77)
    slots = np.array([7, 2, -1, 0, 9, 4], dtype=np.int32)
    pool[2] = 0.0  # sequence 1's slot: zero state
    w = _weight(128)
    note("decode norm state_slots")
    d = device_inputs(inp)
    state = torch.from_numpy(pool).cuda()
    out = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                          state_slots=torch.from_numpy(slots).cuda(),
                          norm_weight=torch.from_numpy(w).cuda(), norm_eps=1e-6)
    torch.cuda.synchronize()
    wd = inp.widened()
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"],
                                      pool[np.maximum(slots, 0)].astype(np.float64))
    y_ref = oracle.rms_norm(o_ref, w, 1e-6)
    got = to_f64(state)
    y = to_f64(out)
    assert np.all(y[1] == 0) and np.all(y_ref[1] == 0)
    for b, s in enumerate(slots):
        if s < 0:
            assert np.all(y[b] == 0)
            continue
        assert rel_err(y[b], y_ref[b]) <= 2e-2
        assert rel_err(got[s], s_ref[b]) <= TOL_F32
    for s in set(range(slots_n)) - set(int(x) for x in slots):
        assert np.array_equal(got[s], pool[s].astype(np.float64))


def _prefill_norm(inp, *, chunk, w, eps, scale=1.0, cu=None, s0=None):
    d = device_inputs(inp)
    T, hv, dv = inp.total_tokens, inp.hv, inp.dv
    out_dtype = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    out = torch.full((T, hv, dv), float("nan"), dtype=out_dtype, device="cuda")
    n = inp.num_seqs if cu is None else cu.numel() - 1
    fin = torch.full((n, hv, dv, inp.dk), float("nan"), dtype=torch.float32, device="cuda")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"] if cu is None else cu,
                       chunk=chunk, scale=scale,
                       initial_state=d["initial_state"] if s0 is None else s0, final_state=fin, out=out,
                       norm_weight=torch.from_numpy(w).cuda(), norm_eps=eps)
    torch.cuda.synchronize()
    return o, f


@pytest.mark.parametrize("chunk", [64, 16, 1])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prefill_norm_ragged(chunk, io):
    """Ragged sequences with an empty one, initial states, scale; chunked and
    token by token."""
    inp = gs.make_inputs([1, 70, 0, 130, 33], 2, 4, 64, 64, seed=81, io_dtype=io, gate_dtype="f32",
                         init_state=True)
    w = _weight(64)
    note(f"prefill norm ragged chunk={chunk} io={io}")
    o, f = _prefill_norm(inp, chunk=chunk, w=w, eps=0.05, scale=0.75)
    o_ref, f_ref = oracle_ref(inp, scale=0.75)
    y_ref = oracle.rms_norm(o_ref, w, 0.05)
    y = to_f64(o)
    eo, ef = rel_err(y, y_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] prefill norm ragged chunk={chunk} io={io} out_err={eo:.3e} state_err={ef:.3e}",
          flush=True)
    assert np.isfinite(y).all()
    assert eo <= tol(io) and ef <= tol(io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 128])
def test_prefill_norm_head_sizes(d, io):
    """fp32: the pass after the scan. bf16: fused into the scan; at d = 16
    the 16-row slices hold whole rows (normalised in the output waves), at
    d = 32 and 128 two and eight slices exchange partial sums."""
    inp = gs.make_inputs([45, 100], 2, 4, d, d, seed=83 + d, io_dtype=io, gate_dtype="f32",
                         init_state=True)
    w = _weight(d, seed=d)
    note(f"prefill norm d={d} io={io}")
    o, f = _prefill_norm(inp, chunk=32, w=w, eps=1e-6)
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o), oracle.rms_norm(o_ref, w, 1e-6)) <= tol(io)
    assert rel_err(to_f64(f), f_ref) <= tol(io)


@pytest.mark.parametrize("chunk", [64, 1])
def test_prefill_norm_4k(chunk):
    """The prefill workload (T = 4096, HK = 16, HV = 32, d = 128, bf16), every
    value head; the final state is the plain call's, bit for bit."""
    inp = gs.workload("prefill", io_dtype="bf16")
    w = _weight(128)
    note(f"prefill norm T=4096 chunk={chunk}")
    o, f = _prefill_norm(inp, chunk=chunk, w=w, eps=1e-6)
    o_ref, f_ref = oracle_ref(inp)
    y_ref = oracle.rms_norm(o_ref, w, 1e-6)
    eo = rel_err(to_f64(o), y_ref)
    print(f"[parity] prefill norm T=4096 chunk={chunk} out_err={eo:.3e}", flush=True)
    assert eo <= tol("bf16")
    d = device_inputs(inp)
    note(f"plain prefill T=4096 chunk={chunk}")
    _, f_plain = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(f, f_plain)


def test_prefill_norm_leaves_rows_outside_sequences():
    """cu_seqlens[0] > 0: rows of the tokens before the first sequence are not
    written by the normalisation pass either."""
    inp = gs.make_inputs([5, 70, 33], 2, 4, 32, 32, seed=43, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    w = _weight(32)
    d = device_inputs(inp)
    cu = d["cu_seqlens"][1:].contiguous()
    note("prefill norm with cu_seqlens[0] = 5")
    o, f = _prefill_norm(inp, chunk=16, w=w, eps=1e-6, cu=cu, s0=d["initial_state"][1:].contiguous())
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o)[5:], oracle.rms_norm(o_ref[5:], w, 1e-6)) <= tol("bf16")
    assert rel_err(to_f64(f), f_ref[1:]) <= tol("bf16")
    assert torch.isnan(o[:5].float()).all()


@pytest.mark.parametrize("lens,io,rows", [([700, 333], "bf16", 32), ([200] * 3, "bf16", 64),
                                          ([200] * 8, "bf16", 128), ([200] * 40, "bf16", 128),
                                          ([200] * 3, "f32", 16)])
def test_prefill_norm_slices_and_passes(lens, io, rows):
    """HK = 16, HV = 32, d = 128. bf16, two or three sequences: 32- or 64-row
    scan slices (4 or 2 per head), one pass over the GPU, so the
    normalisation is fused into the scan, the slices of a head exchanging
    their partial sums. bf16, eight or forty sequences: 128-row slices, each
    one head's whole state, which normalise their own rows in the scan (forty:
    five passes over the GPU). fp32, three sequences: 16-row slices, more
    scan workgroups than one pass holds, so a pass over out normalises after
    the scan. All against the oracle, with the plain call's final states bit
    for bit."""
    io_dtype = torch.bfloat16 if io == "bf16" else torch.float32
    assert gdn.prefill_plan(len(lens), sum(lens), 16, 32, 128, 64, io_dtype) == (64, rows)
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 520 + len(lens), io_dtype=io,
                         gate_dtype="f32", init_state=True)
    w = _weight(128, seed=9)
    note(f"prefill norm lens={lens} io={io} rows={rows}")
    o, f = _prefill_norm(inp, chunk=64, w=w, eps=1e-6)
    o_ref, f_ref = oracle_ref(inp)
    eo = rel_err(to_f64(o), oracle.rms_norm(o_ref, w, 1e-6))
    print(f"[parity] prefill norm lens={lens} io={io} out_err={eo:.3e}", flush=True)
    assert np.isfinite(to_f64(o)).all() and eo <= tol(io)
    d = device_inputs(inp)
    _, f_plain = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                             initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(f, f_plain)


def test_prefill_norm_repeated_calls_are_identical():
    """The fused normalisation sums the row slices' partials in a fixed
    order, so repeated calls give the same bits; a call after one with other
    inputs (the partial slots then hold old values until the preparation
    kernel resets them) too."""
    inp = gs.workload("prefill", io_dtype="bf16")
    other = gs.make_inputs([4096], 16, 32, 128, 128, seed=gs.SEED_BASE + 531, io_dtype="bf16",
                           gate_dtype="f32")
    w = torch.from_numpy(_weight(128)).cuda()
    d, e = device_inputs(inp), device_inputs(other)
    ws = torch.empty(gdn.prefill_workspace_size(1, 4096, 16, 32, 128, 128, 64, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    note("prefill norm repeated")
    outs = []
    for x in (d, d, e, d):
        o, _ = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], chunk=64,
                           norm_weight=w, norm_eps=1e-6, workspace=ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[3])
    assert not torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("lens,rows", [([300, 77, 5], 64), ([700, 5], 32)])
def test_prefill_norm_slice_waits_for_partner(lens, rows):
    """Ragged batches with a 5-token sequence: 64- or 32-row slices (two or
    four per head) that exchange partial sums. The short sequence's slices
    finish their one chunk in a few steps, so one of a head's slices often
    reaches the sum before its partners have published (most often in the
    first calls of a process, on fresh memory) and retries its loads until
    the partials arrive. Four inputs, each called three times with freshly
    allocated outputs, in the order a serving loop would: every call finite,
    the same bits on every repeat, and the oracle's values."""
    n = len(lens)
    assert gdn.prefill_plan(n, sum(lens), 16, 32, 128, 64) == (64, rows)
    w = _weight(128, seed=11)
    wt = torch.from_numpy(w).cuda()
    inps = [gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 540 + 10 * n + i, io_dtype="bf16",
                           gate_dtype="f32", init_state=True) for i in range(4)]
    devs = [device_inputs(x) for x in inps]
    ws = torch.empty(gdn.prefill_workspace_size(n, sum(lens), 16, 32, 128, 128, 64, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    note(f"prefill norm slice waits lens={lens}: 4 inputs x 3 calls")
    outs = [[] for _ in inps]
    for rep in range(3):
        for i, d in enumerate(devs):
            o, _ = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                               initial_state=d["initial_state"],
                               final_state=torch.empty((n, 32, 128, 128), dtype=torch.float32, device="cuda"),
                               out=torch.empty((sum(lens), 32, 128), dtype=torch.bfloat16, device="cuda"),
                               norm_weight=wt, norm_eps=1e-6, workspace=ws)
            torch.cuda.synchronize()
            outs[i].append(o)
    for i, inp in enumerate(inps):
        for rep, o in enumerate(outs[i]):
            nan = int(torch.isnan(o.float()).sum())
            assert nan == 0, f"input {i} call {rep}: {nan} NaN outputs (a slice gave up waiting)"
            assert torch.equal(o, outs[i][0]), f"input {i} call {rep} differs from its first call"
        o_ref, _ = oracle_ref(inp)
        eo = rel_err(to_f64(outs[i][0]), oracle.rms_norm(o_ref, w, 1e-6))
        print(f"[parity] prefill norm slice waits input {i} out_err={eo:.3e}", flush=True)
        assert eo <= tol("bf16")


def test_prefill_norm_exchange_on_concurrent_streams():
    """Slices of a head that exchange partial sums must all be resident at
    once. Two prefills that each fill the GPU (one 4,096-token sequence,
    16-row slices: 256 workgroups) run on two streams at once, beside a long
    matrix product on a third; the slices of each head sit next to one
    another in an XCD's dispatch order, so every call still finishes without
    exhausting its wait. Every output equals that of the same call made
    alone, bit for bit."""
    lens = [4096]
    assert gdn.prefill_plan(1, 4096, 16, 32, 128, 64) == (64, 16)
    w = torch.from_numpy(_weight(128, seed=12)).cuda()
    inps = [device_inputs(gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 560 + i,
                                         io_dtype="bf16", gate_dtype="f32")) for i in range(2)]
    size = gdn.prefill_workspace_size(1, 4096, 16, 32, 128, 128, 64, torch.bfloat16)
    wss = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(2)]

    def call(i, stream=None):
        d = inps[i]
        o, _ = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                           norm_weight=w, norm_eps=1e-6, workspace=wss[i], stream=stream)
        return o

    note("prefill norm exchange: alone")
    alone = [call(0), call(1)]
    torch.cuda.synchronize()
    a = torch.randn(4096, 4096, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    main = torch.cuda.current_stream()
    for st in streams:
        st.wait_stream(main)
    note("prefill norm exchange: two streams and a matrix product")
    outs = []
    for rep in range(4):
        with torch.cuda.stream(streams[2]):
            a = (a @ a).clamp_(-1.0, 1.0)
        outs.append((call(0, streams[0]), call(1, streams[1])))
    for st in streams:
        main.wait_stream(st)
    torch.cuda.synchronize()
    for rep, (o0, o1) in enumerate(outs):
        assert not torch.isnan(o0.float()).any() and not torch.isnan(o1.float()).any(), f"rep {rep}: NaN rows"
        assert torch.equal(o0, alone[0]) and torch.equal(o1, alone[1]), f"rep {rep}: differs from the call alone"


def test_prefill_norm_on_a_cu_masked_stream():
    """A stream whose CU mask leaves out one CU in every 32 cannot be
    counted on to hold a GPU-filling exchanging scan at once, so a 4,096-token
    prefill with the norm on it normalises in the pass after the scan (one
    norm_apply launch), and meets the oracle's bar; on the default stream the
    same call fuses the norm into the scan."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (ncu + 31) // 32
    mask = (ctypes.c_uint32 * words)(*([0xFFFFFFFE] * words))
    inp = gs.workload("prefill", io_dtype="bf16")
    w = _weight(128, seed=13)
    d = device_inputs(inp)
    wt = torch.from_numpy(w).cuda()

    def call(stream):
        gdn.timing_start(8)
        o, _ = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                           norm_weight=wt, norm_eps=1e-6, stream=stream)
        kt = gdn.timing_stop()
        torch.cuda.synchronize()
        return o, kt["norm_apply"]["count"]

    note("prefill norm on the default stream")
    o_fused, passes = call(None)
    assert passes == 0
    handle = ctypes.c_void_p()
    assert hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), words, mask) == 0
    try:
        st = torch.cuda.ExternalStream(handle.value)
        st.wait_stream(torch.cuda.current_stream())
        note("prefill norm on a CU-masked stream")
        o_masked, passes = call(st)
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(handle)
    assert passes == 1
    o_ref, _ = oracle_ref(inp)
    y_ref = oracle.rms_norm(o_ref, w, 1e-6)
    for o in (o_fused, o_masked):
        eo = rel_err(to_f64(o), y_ref)
        print(f"[parity] prefill norm masked-stream case out_err={eo:.3e}", flush=True)
        assert np.isfinite(to_f64(o)).all() and eo <= tol("bf16")


@pytest.mark.parametrize("hk,hv,d", [(4, 16, 64), (8, 8, 128), (2, 8, 32)])
def test_prefill_norm_whole_head_slices(hk, hv, d):
    """bf16, enough sequences that the scan takes slices of a whole head
    (rows = d, more than one pass over the GPU): each output wave normalises
    its rows itself. Against the oracle (an empty sequence among them), with
    the plain call's final states bit for bit."""
    n = 40
    assert gdn.prefill_plan(n, n * 90, hk, hv, d, 64) == (64, d)
    rng = np.random.default_rng(hk + hv + d)
    lens = [int(x) for x in rng.integers(1, 180, size=n)]
    lens[5] = 0
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=gs.SEED_BASE + 540 + d, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    w = _weight(d, seed=d + 1)
    note(f"prefill norm whole-head slices hk={hk} hv={hv} d={d}")
    o, f = _prefill_norm(inp, chunk=64, w=w, eps=1e-6, scale=0.9)
    o_ref, f_ref = oracle_ref(inp, scale=0.9)
    eo = rel_err(to_f64(o), oracle.rms_norm(o_ref, w, 1e-6))
    print(f"[parity] prefill norm whole-head slices hk={hk} hv={hv} d={d} out_err={eo:.3e}", flush=True)
    assert np.isfinite(to_f64(o)).all() and eo <= tol("bf16")
    dd = device_inputs(inp)
    _, f_plain = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"], chunk=64,
                             scale=0.9, initial_state=dd["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(f, f_plain)


@pytest.mark.parametrize("rows_case", ["whole_head", "exchanging"])
def test_prefill_norm_bf16_states(rows_case):
    """bf16 state storage with the normalisation fused into the scan: 40
    sequences (128-row slices, whole rows per output wave) and 3 sequences
    (64-row slices, two per head exchanging partial sums). Against the oracle
    started from the bf16-rounded initial state; the final state is the
    plain call's, bit for bit."""
    n = 40 if rows_case == "whole_head" else 3
    rows = 128 if rows_case == "whole_head" else 64
    hk, hv, d = (8, 8, 128) if rows_case == "whole_head" else (16, 32, 128)
    assert gdn.prefill_plan(n, n * 120, hk, hv, d, 64) == (64, rows)
    rng = np.random.default_rng(77 + n)
    lens = [int(x) for x in rng.integers(1, 240, size=n)]
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=gs.SEED_BASE + 560 + n, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    w = _weight(d, seed=3)
    dd = device_inputs(inp)
    s0 = dd["initial_state"].to(torch.bfloat16)
    note(f"prefill norm bf16 states {rows_case} n={n}")
    wt = torch.from_numpy(w).cuda()
    o, f = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"], chunk=64,
                       initial_state=s0, state_dtype=torch.bfloat16, norm_weight=wt, norm_eps=1e-6)
    _, f_plain = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"], chunk=64,
                             initial_state=s0, state_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_ref(inp, initial_state=to_f64(s0))
    eo = rel_err(to_f64(o), oracle.rms_norm(o_ref, w, 1e-6))
    ef = rel_err(to_f64(f), f_ref)
    print(f"[parity] prefill norm bf16 states {rows_case} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert np.isfinite(to_f64(o)).all() and eo <= tol("bf16") and ef <= tol("bf16")
    assert torch.equal(f, f_plain)
