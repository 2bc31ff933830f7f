"""Head layouts other than two value heads per query/key head, against the
fp64 oracle: one query/key head shared by every value head (hk = 1), groups
of 4 and 8 (past the two value heads whose gates the preparation kernel
prefetches), and one value head per query/key head. Chunked, token by token,
and decode; bars as elsewhere (bf16 2e-2, fp32 1e-4 max-rel).
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
import oracle
from gpu_util import device_inputs, note, oracle_ref, rel_err, requires_gpu, run_prefill, to_f64, tol

pytestmark = [pytest.mark.gpu, requires_gpu]

LAYOUTS = [(1, 4), (2, 8), (2, 16), (4, 4)]


@pytest.mark.parametrize("chunk", [64, 16, 1])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("hk,hv", LAYOUTS)
def test_prefill_head_layouts(hk, hv, io, chunk):
    inp = gs.make_inputs([70, 0, 131, 9], hk, hv, 64, 64, seed=1100 + 10 * hk + hv, io_dtype=io,
                         gate_dtype="f32", init_state=True)
    note(f"prefill hk={hk} hv={hv} io={io} chunk={chunk}")
    o, f = run_prefill(inp, chunk=chunk, scale=0.5)
    o_ref, f_ref = oracle_ref(inp, scale=0.5)
    eo, ef = rel_err(to_f64(o), o_ref), rel_err(to_f64(f), f_ref)
    print(f"[parity] heads hk={hk} hv={hv} io={io} chunk={chunk} out_err={eo:.3e} state_err={ef:.3e}",
          flush=True)
    assert np.isfinite(to_f64(o)).all()
    assert eo <= tol(io) and ef <= tol(io)


@pytest.mark.parametrize("hk,hv", LAYOUTS)
def test_decode_head_layouts(hk, hv):
    batch = 5
    inp = gs.make_inputs([1] * batch, hk, hv, 128, 128, seed=1200 + 10 * hk + hv, io_dtype="bf16",
                         gate_dtype="bf16")
    s0 = gs.decode_state(batch, hv, 128, 128, seed=1300 + hv)
    note(f"decode hk={hk} hv={hv}")
    d = device_inputs(inp)
    state = torch.from_numpy(s0).cuda()
    out = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    w = inp.widened()
    o_ref, s_ref = oracle.decode_step(w["q"], w["k"], w["v"], w["g"], w["beta"], s0.astype(np.float64))
    assert rel_err(to_f64(out), o_ref) <= tol("bf16")
    assert rel_err(to_f64(state), s_ref) <= 1e-4
