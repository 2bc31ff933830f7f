"""The kernels' fp32 -> bf16 output rounding, bit for bit, on the GPU.

With a = 1 (g = 0), b = 0 and a standard-basis query e_j, a decode step
writes o_i = S_ij exactly (every other product is an exact zero), rounded to
bf16 by the kernel. Filling column j of the states with chosen fp32 bit
patterns therefore exposes the device's rounding of each pattern; it must
equal round-to-nearest-even as the input generator computes it (itself
checked against numpy exhaustively): every sign/exponent/mantissa high half
with each class of low half rounding can see (zero, smallest, just below the
tie, the tie, just above, largest, and two more), finite values only.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_output_rounding_is_round_to_nearest_even():
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]  # 2^19 patterns minus the non-finite ones
    # -0 reaches the output as +0: the dot product starts from +0, and
    # -0 + 0 = +0 (a property of the sum, not of the rounding)
    vals = vals[~((vals == 0) & np.signbit(vals))]
    B, hk, hv, d, j = 128, 32, 32, 128, 5
    n_rows = B * hv * d
    col = np.zeros(n_rows, dtype=np.float32)
    col[:len(vals)] = vals
    state = np.zeros((B, hv, d, d), dtype=np.float32)
    state[:, :, :, j] = col.reshape(B, hv, d)
    q = np.zeros((B, hk, d), dtype=np.float32)
    q[:, :, j] = 1.0
    bf = lambda x: torch.from_numpy(gs.f32_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)).view(
        torch.bfloat16).cuda()
    dq, dk = bf(q), bf(np.zeros_like(q))
    dv = bf(np.zeros((B, hv, d)))
    dg, db = bf(np.zeros((B, hv))), bf(np.zeros((B, hv)))
    note(f"output rounding of {len(vals)} fp32 patterns")
    st = torch.from_numpy(state).cuda()
    out = gdn.decode_step(dq, dk, dv, dg, db, st)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)[:len(vals)]
    want = gs.f32_to_bf16_bits(vals)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, f"{len(bad)} patterns rounded differently, first {vals[bad[:4]]}"
    # the state came back untouched (a = 1, u = 0)
    assert torch.equal(st, torch.from_numpy(state).cuda())
