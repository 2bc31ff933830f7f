"""The decode step and the prefill captured in a HIP graph (torch.cuda.graph)
and replayed: serving loops capture the per-token step to save launch time.
The library's launch path allocates nothing, sets no memory and never
synchronises, so a captured call must replay exactly as it runs eagerly.
Each replay is checked against the eager result of the same inputs, with
the program's own eager work and synchronisations between the replays.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import device_inputs, note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("norm", [False, True])
def test_decode_step_graph_replays(norm, state_dtype):
    B, hk, hv, d = 8, 16, 32, 128
    w = torch.from_numpy(gs.norm_weight(d, seed=gs.SEED_BASE + 505)).cuda() if norm else None
    steps = [device_inputs(gs.make_inputs([1] * B, hk, hv, d, d, seed=gs.SEED_BASE + 1400 + t,
                                          io_dtype="bf16", gate_dtype="bf16")) for t in range(5)]
    s0 = torch.from_numpy(gs.decode_state(B, hv, d, d, seed=gs.SEED_BASE + 1500)).cuda().to(state_dtype)
    # static buffers the graph reads and writes
    sq, sk, sv, sg, sb = (steps[0][x].clone() for x in ("q", "k", "v", "g", "beta"))
    state = s0.clone()
    out = torch.empty((B, hv, d), dtype=torch.bfloat16, device="cuda")
    note(f"decode graph capture norm={norm} state={state_dtype}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        gdn.decode_step(sq, sk, sv, sg, sb, state.clone(), out=out, norm_weight=w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.decode_step(sq, sk, sv, sg, sb, state, out=out, norm_weight=w)
    # replay token by token; the eager reference advances its own state copy
    ref_state = s0.clone()
    state.copy_(s0)
    for t in range(1, 5):
        for name, buf in zip(("q", "k", "v", "g", "beta"), (sq, sk, sv, sg, sb)):
            buf.copy_(steps[t][name])
        note(f"decode graph replay {t}")
        graph.replay()
        ref_out = gdn.decode_step(steps[t]["q"], steps[t]["k"], steps[t]["v"], steps[t]["g"], steps[t]["beta"],
                                  ref_state, norm_weight=w)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {t}: outputs differ from the eager call"
        assert torch.equal(state, ref_state), f"replay {t}: states differ from the eager call"


@pytest.mark.parametrize("lens,norm,rows,hint", [([300, 77, 5], False, 64, None), ([300, 77, 5], True, 64, None),
                                                ([120, 7, 64, 200] * 3, True, 128, None),
                                                ([2048, 256, 256, 256, 256], True, 32, 2048)])
def test_prefill_graph_replays(lens, norm, rows, hint):
    """Chunked prefill (preparation and scan), captured once and replayed on
    new token data; every replay equals the eager call. 3 sequences take
    64-row scan slices (with a normalisation weight their slices exchange
    partial sums through the workspace, whose slots the preparation kernel
    resets in every replay); 12 take 128-row slices, normalised in place;
    an uneven batch given its longest length (max_seqlen) takes 32-row
    slices rather than the rule's 128."""
    assert gdn.prefill_plan(len(lens), sum(lens), 16, 32, 128, 64, max_seqlen=hint) == (64, rows)
    runs = [gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 1600 + t, io_dtype="bf16",
                           gate_dtype="f32", init_state=True) for t in range(4)]
    w = torch.from_numpy(gs.norm_weight(128, seed=gs.SEED_BASE + 1650)).cuda() if norm else None
    dev = [device_inputs(r) for r in runs]
    T, N = sum(lens), len(lens)
    static = {x: dev[0][x].clone() for x in ("q", "k", "v", "g", "beta", "cu_seqlens", "initial_state")}
    out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, 32, 128, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_size(N, T, 16, 32, 128, 128, 64, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")

    def call(src, o, f):
        return gdn.prefill(src["q"], src["k"], src["v"], src["g"], src["beta"], src["cu_seqlens"], chunk=64,
                           initial_state=src["initial_state"], final_state=f, out=o, workspace=ws,
                           norm_weight=w, norm_eps=1e-6, max_seqlen=hint)

    note(f"prefill graph capture lens={lens[:4]} norm={norm} hint={hint}")
    call(static, out, fin)  # warm-up (first launch sets kernel attributes)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, out, fin)
    for t in range(1, 4):
        for x in static:
            static[x].copy_(dev[t][x])
        note(f"prefill graph replay {t}")
        graph.replay()
        torch.cuda.synchronize()
        o_g, f_g = out.clone(), fin.clone()
        o_e, f_e = call(dev[t], torch.empty_like(out), torch.empty_like(fin))
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(f_g, f_e), f"replay {t} differs from the eager call"
