"""Seeded random configurations against the fp64 oracle: sequence counts
and lengths (empty and ragged ones included), head layouts, head sizes,
dtypes, methods (chunk 0, 1, 16, 32, 64), scale, initial states or none,
and gates with occasional extreme decays (g = -1e4, a = 0) and b = 0 or 1.
Every case is drawn from its own seed, printed before it runs, and held to
the usual bars (bf16 2e-2, fp32 1e-4 max-rel). A second set draws batches
large enough that the chunked scan takes 32 state rows per workgroup
(N * HV * DV / 16 > 256, bf16 I/O). A third set adds the output
normalisation (a weight per value channel and eps) to random ragged
batches with short and empty sequences, against oracle.rms_norm of the
oracle's output, whichever form the call takes (in-wave, exchanged between
row slices, or the pass after the scan). A fourth draws decode steps: batch, head
layout and size, I/O and gate dtypes, scale, state slots (permuted, some
skipped with -1), the fused normalisation, and fp32 or (with bf16 I/O) bf16
state storage; skipped slots must keep their bits and give rows of zeros.
A fifth draws uneven bf16 batches called with the longest length as the
method rule's hint (max_seqlen), against the oracle."""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle
from gpu_util import TOL_BF16, TOL_F32, device_inputs, note, oracle_ref, rel_err, requires_gpu, run_prefill, to_f64, tol

pytestmark = [pytest.mark.gpu, requires_gpu]

LAYOUTS = [(1, 1), (1, 2), (2, 4), (2, 2), (4, 8), (1, 8), (4, 4)]


def _case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 260, n)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, n))] = 0
    hk, hv = LAYOUTS[int(rng.integers(0, len(LAYOUTS)))]
    d = int(rng.choice([16, 32, 64, 128]))
    io = "bf16" if rng.random() < 0.5 else "f32"
    gate = "bf16" if (io == "bf16" and rng.random() < 0.5) else "f32"
    chunk = int(rng.choice([0, 1, 16, 32, 64]))
    scale = float(rng.choice([1.0, 0.5, 1.0 / np.sqrt(d)]))
    init = bool(rng.random() < 0.6)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=seed, io_dtype=io, gate_dtype=gate, init_state=init)
    # occasional extreme gates: decays that underflow, no writes, full writes
    g = gs.widen(inp.g, gate)
    b = gs.widen(inp.beta, gate)
    extreme = rng.random(g.shape)
    g = np.where(extreme < 0.03, -1e4, g)
    b = np.where(extreme > 0.97, 0.0, np.where((extreme > 0.94) & (extreme <= 0.97), 1.0, b))
    inp.g = gs.to_storage(g, gate)
    inp.beta = gs.to_storage(b, gate)
    desc = f"seed={seed} lens={lens} hk={hk} hv={hv} d={d} io={io} gate={gate} chunk={chunk} scale={scale:.3f} init={init}"
    return inp, chunk, scale, desc


@pytest.mark.parametrize("seed", range(5000, 5024))
def test_random_configuration(seed):
    inp, chunk, scale, desc = _case(seed)
    note(desc)
    o, f = run_prefill(inp, chunk=chunk, scale=scale)
    o_ref, f_ref = oracle_ref(inp, scale=scale)
    og, fg = to_f64(o), to_f64(f)
    assert np.isfinite(og).all() and np.isfinite(fg).all(), desc
    eo = rel_err(og, o_ref) if og.size else 0.0
    ef = rel_err(fg, f_ref)
    print(f"[parity] random {desc} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(inp.io_dtype) and ef <= tol(inp.io_dtype), desc


def _wide_case(seed):
    rng = np.random.default_rng(seed)
    hk, hv = [(2, 8), (4, 16), (8, 32), (16, 48)][int(rng.integers(0, 4))]
    d = int(rng.choice([32, 64, 128]))
    one_pass = 256 // (hv * d // 16)
    n = int(rng.integers(one_pass + 1, one_pass + 12))
    lens = [int(x) for x in rng.integers(0, 200, n)]
    chunk = int(rng.choice([0, 16, 32, 64]))
    init = bool(rng.random() < 0.7)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=seed, io_dtype="bf16", gate_dtype="f32", init_state=init)
    desc = f"seed={seed} n={n} hk={hk} hv={hv} d={d} chunk={chunk} init={init} T={sum(lens)}"
    return inp, chunk, desc


@pytest.mark.parametrize("seed", range(7000, 7012))
def test_random_wide_batch(seed):
    inp, chunk, desc = _wide_case(seed)
    note(f"wide {desc}")
    o, f = run_prefill(inp, chunk=chunk)
    o_ref, f_ref = oracle_ref(inp)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] random wide {desc} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol("bf16") and ef <= tol("bf16"), desc


def _norm_case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 300, n)]
    for i in range(n):  # short sequences: one partial chunk, done in a few steps
        if rng.random() < 0.35:
            lens[i] = int(rng.integers(0, 9))
    hk, hv = [(16, 32), (8, 16), (4, 8), (2, 4), (1, 2)][int(rng.integers(0, 5))]
    d = int(rng.choice([16, 32, 64, 128]))
    io = "bf16" if rng.random() < 0.75 else "f32"
    chunk = int(rng.choice([0, 0, 1, 16, 32, 64]))
    eps = float(rng.choice([1e-6, 1e-3, 0.05]))
    init = bool(rng.random() < 0.6)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=seed, io_dtype=io, gate_dtype="f32", init_state=init)
    w = gs.norm_weight(d, seed=seed + 1)
    desc = f"seed={seed} lens={lens} hk={hk} hv={hv} d={d} io={io} chunk={chunk} eps={eps} init={init}"
    return inp, chunk, w, eps, desc


@pytest.mark.parametrize("seed", range(9000, 9016))
def test_random_normalised_configuration(seed):
    inp, chunk, w, eps, desc = _norm_case(seed)
    io_dtype = torch.bfloat16 if inp.io_dtype == "bf16" else torch.float32
    plan = gdn.prefill_plan(inp.num_seqs, max(inp.total_tokens, 1), inp.hk, inp.hv, inp.dk, chunk, io_dtype)
    note(f"norm {desc} plan={plan}")
    o, f = run_prefill(inp, chunk=chunk, norm_weight=torch.from_numpy(w).cuda(), norm_eps=eps)
    o_ref, f_ref = oracle_ref(inp)
    y_ref = oracle.rms_norm(o_ref, w, eps)
    og, fg = to_f64(o), to_f64(f)
    assert np.isfinite(og).all() and np.isfinite(fg).all(), desc
    eo = rel_err(og, y_ref) if og.size else 0.0
    ef = rel_err(fg, f_ref)
    print(f"[parity] random norm {desc} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= tol(inp.io_dtype) and ef <= tol(inp.io_dtype), desc


def _decode_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 65))
    hk, hv = LAYOUTS[int(rng.integers(0, len(LAYOUTS)))]
    d = int(rng.choice([16, 32, 64, 128]))
    io = "bf16" if rng.random() < 0.6 else "f32"
    gate = "bf16" if (io == "bf16" and rng.random() < 0.6) else "f32"
    state_bf16 = bool(io == "bf16" and rng.random() < 0.4)  # bf16 storage is built for bf16 I/O only
    norm = bool(rng.random() < 0.4)
    eps = float(rng.choice([1e-6, 0.05]))
    scale = float(rng.choice([1.0, 1.0 / np.sqrt(d)]))
    inp = gs.make_inputs([1] * B, hk, hv, d, d, seed=seed, io_dtype=io, gate_dtype=gate)
    pool_n = B + int(rng.integers(0, 5))
    pool = gs.decode_state(pool_n, hv, d, d, seed=seed + 1)
    if state_bf16:
        pool = oracle.round_to_bf16(pool).astype(np.float32)
    slots = None
    if rng.random() < 0.5:
        slots = rng.permutation(pool_n)[:B].astype(np.int32)
        slots[rng.random(B) < 0.15] = -1
    w = gs.norm_weight(d, seed=seed + 2) if norm else None
    desc = (f"seed={seed} B={B} hk={hk} hv={hv} d={d} io={io} gate={gate} state={'bf16' if state_bf16 else 'f32'} "
            f"norm={norm} eps={eps} scale={scale:.3f} slots={'yes' if slots is not None else 'no'}")
    return inp, pool, slots, state_bf16, w, eps, scale, desc


@pytest.mark.parametrize("seed", range(9500, 9516))
def test_random_decode_step(seed):
    inp, pool, slots, state_bf16, w, eps, scale, desc = _decode_case(seed)
    note(f"decode {desc}")
    d = device_inputs(inp)
    pool_t = torch.from_numpy(pool).cuda()
    state = pool_t.to(torch.bfloat16) if state_bf16 else pool_t.clone()
    out = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, scale=scale,
                          state_slots=None if slots is None else torch.from_numpy(slots).cuda(),
                          norm_weight=None if w is None else torch.from_numpy(w).cuda(), norm_eps=eps)
    torch.cuda.synchronize()
    wd = inp.widened()
    idx = np.arange(inp.num_seqs) if slots is None else np.maximum(slots, 0)
    o_ref, s_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"],
                                      pool[idx].astype(np.float64), scale=scale)
    if w is not None:
        o_ref = oracle.rms_norm(o_ref, w, eps)
    o, got = to_f64(out), to_f64(state)
    live = np.ones(inp.num_seqs, bool) if slots is None else slots >= 0
    assert np.isfinite(o).all() and np.isfinite(got).all(), desc
    assert np.all(o[~live] == 0), desc
    eo = rel_err(o[live], o_ref[live]) if live.any() else 0.0
    s_bar = TOL_BF16 if state_bf16 else TOL_F32
    es = rel_err(got[idx[live]], s_ref[live]) if live.any() else 0.0
    untouched = sorted(set(range(pool.shape[0])) - set(int(x) for x in idx[live]))
    print(f"[parity] random decode {desc} out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= tol(inp.io_dtype) and es <= s_bar, desc
    assert np.array_equal(got[untouched], pool[untouched].astype(np.float64)), desc


def _hint_case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 9))
    lens = [int(x) for x in rng.integers(1, 400, n)]
    lens[int(rng.integers(0, n))] = int(rng.integers(400, 1500))  # one long sequence
    hk, hv = [(16, 32), (8, 16), (4, 8), (2, 4)][int(rng.integers(0, 4))]
    d = int(rng.choice([32, 64, 128]))
    init = bool(rng.random() < 0.6)
    inp = gs.make_inputs(lens, hk, hv, d, d, seed=seed, io_dtype="bf16", gate_dtype="f32", init_state=init)
    desc = f"seed={seed} lens={lens} hk={hk} hv={hv} d={d} init={init}"
    return inp, desc


@pytest.mark.parametrize("seed", range(9700, 9712))
def test_random_hinted_configuration(seed):
    inp, desc = _hint_case(seed)
    lens = np.diff(inp.cu_seqlens)
    hint = int(lens.max())
    plan = gdn.prefill_plan(inp.num_seqs, inp.total_tokens, inp.hk, inp.hv, inp.dk, max_seqlen=hint)
    note(f"hinted {desc} plan={plan}")
    o, f = run_prefill(inp, chunk=0, max_seqlen=hint)
    o_ref, f_ref = oracle_ref(inp)
    og, fg = to_f64(o), to_f64(f)
    assert np.isfinite(og).all() and np.isfinite(fg).all(), desc
    eo, ef = rel_err(og, o_ref), rel_err(fg, f_ref)
    print(f"[parity] random hinted {desc} plan={plan} out_err={eo:.3e} state_err={ef:.3e}", flush=True)
    assert eo <= TOL_BF16 and ef <= TOL_BF16, desc
