"""States stored in bf16 between calls (gdn_decode_step_ex and gdn_prefill_ex
with state_dtype bf16) against the fp64 oracle.

The variant's definition: every call widens the stored bf16 state, applies
the rule in fp32, and rounds the state it stores to bf16 (nearest even):
after each decode step, and once at the end of a prefill. Its oracle is
oracle.decode_step / oracle.scan on the widened state followed by
oracle.round_to_bf16. Outputs and states are held to the bf16 bar (2e-2
max-rel); besides, at least 99% of the stored state's elements must equal
the oracle's rounded state, and none may be more than one bf16 step (at the
tensor's largest magnitude) away from it.

The accuracy cost against fp32 states (the pages disagree on which to keep)
is measured over 256 decode steps against the exact fp64 recurrence, with
the generator's gates and with no decay at all (g = 0), where rounding
errors are never forgotten.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle
from gpu_util import TOL_BF16, device_inputs, note, rel_err, requires_gpu, to_f64

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bf16_state(x64):
    """fp64 -> bf16 tensor on the GPU (exact when x64 holds bf16 values)."""
    bits = gs.f32_to_bf16_bits(np.asarray(x64, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _check_state(got_bf16, ref64, label):
    """Nearly every element rounds as the oracle's does; the others differ
    where the fp32 result lies within fp32 rounding of a different bf16
    value. Where a S and u k^T nearly cancel, that fp32 error is comparable
    to one bf16 step of the small result itself, so the gap is measured in
    bf16 steps at the tensor's largest magnitude."""
    want = oracle.round_to_bf16(ref64)
    got = to_f64(got_bf16)
    same = float(np.mean(got == want))
    step = float(np.abs(want).max()) * 2.0 ** -7
    worst = float(np.abs(got - want).max()) / step
    print(f"[parity] bf16 state {label}: identical {same:.6f}, worst {worst:.3f} bf16 steps at max, "
          f"max-rel vs unrounded {rel_err(got, ref64):.3e}", flush=True)
    assert same >= 0.99, f"{label}: only {same:.4f} of elements equal the oracle's rounding"
    assert worst <= 1.0, f"{label}: an element is {worst} bf16 steps (at the largest magnitude) away"
    assert rel_err(got, ref64) <= TOL_BF16


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("batch", [1, 64])
def test_decode_bf16_state(batch, norm):
    """The decode workload (HK = 16, HV = 32, d = 128) with a bf16 state pool."""
    inp = gs.make_inputs([1] * batch, 16, 32, 128, 128, seed=gs.SEED_BASE + 1, io_dtype="bf16",
                         gate_dtype="bf16")
    s0 = oracle.round_to_bf16(gs.decode_state(batch, 32, 128, 128, seed=gs.SEED_BASE + 101))
    w = gs.norm_weight(128, seed=gs.SEED_BASE + 505)
    note(f"decode bf16 state batch={batch} norm={norm}")
    d = device_inputs(inp)
    state = _bf16_state(s0)
    out = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                          norm_weight=torch.from_numpy(w).cuda() if norm else None)
    torch.cuda.synchronize()
    wd = inp.widened()
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], s0)
    if norm:
        o_ref = oracle.rms_norm(o_ref, w, 1e-6)
    eo = rel_err(to_f64(out), o_ref)
    print(f"[parity] decode bf16 state B={batch} norm={norm} out_err={eo:.3e}", flush=True)
    assert eo <= TOL_BF16
    _check_state(state, s_ref, f"decode B={batch} norm={norm}")


def test_decode_bf16_state_slots():
    """Indirect slots in a bf16 pool: slot -1 is skipped (zeros out), and
    slots no sequence names keep their bits."""
    batch, slots_n = 6, 10
    inp = gs.make_inputs([1] * batch, 16, 32, 128, 128, seed=gs.SEED_BASE + 6, io_dtype="bf16",
                         gate_dtype="bf16")
    pool = oracle.round_to_bf16(gs.decode_state(slots_n, 32, 128, 128, seed=gs.SEED_BASE + 77))
    slots = np.array([7, 2, -1, 0, 9, 4], dtype=np.int32)
    note("decode bf16 state slots")
    d = device_inputs(inp)
    state = _bf16_state(pool)
    before = state.clone()
    out = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                          state_slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    wd = inp.widened()
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], pool[np.maximum(slots, 0)])
    o = to_f64(out)
    for b, s in enumerate(slots):
        if s < 0:
            assert np.all(o[b] == 0)
            continue
        assert rel_err(o[b], o_ref[b]) <= TOL_BF16
        _check_state(state[s], s_ref[b], f"slot {s}")
    for s in set(range(slots_n)) - set(int(x) for x in slots):
        assert torch.equal(state[s], before[s])


@pytest.mark.parametrize("chunk", [64, 16, 1])
def test_prefill_bf16_state(chunk):
    """Ragged sequences (one empty) from bf16 initial states to bf16 final
    states. The state is widened once and rounded once, at the end, so the
    call must equal the fp32-state call from the same (widened) initial
    state, with its final state rounded to bf16: identical outputs and
    state bits. Against the oracle both meet the bf16 bar; token by token
    (fp32 arithmetic) the stored state also rounds as the oracle's does."""
    inp = gs.make_inputs([1, 70, 0, 130, 33], 2, 4, 64, 64, seed=91, io_dtype="bf16", gate_dtype="f32",
                         init_state=True)
    s0 = oracle.round_to_bf16(inp.initial_state)
    note(f"prefill bf16 state chunk={chunk}")
    d = device_inputs(inp)
    init = _bf16_state(s0)
    fin = torch.full(init.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk, scale=0.75,
                       initial_state=init, final_state=fin)
    o32, f32 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                           scale=0.75, initial_state=init.float())
    torch.cuda.synchronize()
    assert torch.equal(o, o32)
    assert torch.equal(f, f32.to(torch.bfloat16))
    w = inp.widened()
    o_ref, f_ref = oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"], scale=0.75,
                               initial_state=s0)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] prefill bf16 state chunk={chunk} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    if chunk == 1:
        _check_state(f, f_ref, "prefill token by token")
    # the empty sequence passes its state through unchanged
    assert torch.equal(f[2], init[2])


def test_prefill_bf16_state_4k():
    """The prefill workload (T = 4096, HK = 16, HV = 32, d = 128) with a bf16
    final state, every value head; output identical to the fp32-state call
    (the state is rounded only once it is stored)."""
    inp = gs.workload("prefill", io_dtype="bf16")
    note("prefill bf16 state T=4096")
    d = device_inputs(inp)
    o16, f16 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64,
                           state_dtype=torch.bfloat16)
    o32, f32 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=64)
    torch.cuda.synchronize()
    assert f16.dtype == torch.bfloat16
    assert torch.equal(o16, o32)
    assert torch.equal(f16, f32.to(torch.bfloat16))
    w = inp.widened()
    _, f_ref = oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"])
    ef = rel_err(to_f64(f16), f_ref)
    print(f"[parity] prefill bf16 state T=4096 state_err={ef:.3e}", flush=True)
    assert ef <= TOL_BF16


@pytest.mark.parametrize("gates", ["generator", "no_decay"])
def test_bf16_state_error_over_256_decode_steps(gates):
    """256 decode steps of 8 sequences (HK = 16, HV = 32, d = 128, bf16 I/O),
    with fp32 and with bf16 states, against the exact fp64 recurrence. With
    the generator's gates (mean decay 0.7) a rounding error fades within a
    few steps; with g = 0 it is never forgotten and grows like a random walk."""
    B, steps = 8, 256
    s_exact = gs.decode_state(B, 32, 128, 128, seed=gs.SEED_BASE + 131).astype(np.float64)
    s_exact = oracle.round_to_bf16(s_exact)  # both modes start from the same values
    st32 = torch.from_numpy(s_exact.astype(np.float32)).cuda()
    st16 = _bf16_state(s_exact)
    errs = {"f32": [], "bf16": []}
    note(f"256 decode steps gates={gates}")
    for t in range(steps):
        inp = gs.make_inputs([1] * B, 16, 32, 128, 128, seed=gs.SEED_BASE + 1000 + t, io_dtype="bf16",
                             gate_dtype="bf16")
        if gates == "no_decay":
            inp.g[...] = 0  # bf16 bits of +0.0: a = 1
        d = device_inputs(inp)
        o32 = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st32)
        o16 = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st16)
        wd = inp.widened()
        o_ref, s_exact = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], s_exact)
        errs["f32"].append(rel_err(to_f64(o32), o_ref))
        errs["bf16"].append(rel_err(to_f64(o16), o_ref))
    torch.cuda.synchronize()
    s_err = {"f32": rel_err(to_f64(st32), s_exact), "bf16": rel_err(to_f64(st16), s_exact)}
    for m in ("f32", "bf16"):
        e = errs[m]
        print(f"[accuracy] gates={gates} state={m}: out err step1 {e[0]:.3e} step16 {e[15]:.3e} "
              f"step64 {e[63]:.3e} step256 {e[255]:.3e} max {max(e):.3e}; state err after 256 "
              f"{s_err[m]:.3e}", flush=True)
    # fp32 states: the bf16 output rounding alone, flat over the steps
    assert max(errs["f32"]) <= TOL_BF16
    if gates == "generator":
        # the decay forgets each step's rounding: close to the fp32 states
        assert max(errs["bf16"]) <= TOL_BF16
        assert s_err["bf16"] <= TOL_BF16
    else:
        # never forgotten: the error grows with the steps (measured: 5.5e-3
        # after 16, 8e-3 after 64, 1.5e-2 after 256, against a flat 2-3e-3
        # with fp32 states); bounded at twice the measured maximum
        assert errs["bf16"][255] > 3 * errs["f32"][255]
        assert max(errs["bf16"]) <= 0.04
