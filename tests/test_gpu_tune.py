"""Choice of the prefill method by measurement (gdn_tune_prefill) on the GPU.

Every method must pass the correctness gate (its output and final state
within 1/64 of the largest magnitude of the chunk-64 result, the pages' bar)
before it is timed; the fastest passing one is cached, and gdn_prefill with
chunk 0 then runs exactly that method (identical bits to the explicit call,
and the method's kernels in the launch record). Shapes: HK = 16, HV = 32,
d = 128, bf16, from a single short prompt to the 4096-token workload.
"""

import numpy as np
import pytest
import torch

import gdn_synth as gs
import gated_deltanet_linear_02_amd as gdn
from gpu_util import device_inputs, note, oracle_ref, rel_err, requires_gpu, to_f64, tol

pytestmark = [pytest.mark.gpu, requires_gpu]

KERNEL_OF = {1: "token_scan", 16: "scan", 32: "scan", 64: "scan"}


@pytest.fixture(autouse=True)
def empty_cache():
    gdn.tune_cache_clear()
    yield
    gdn.tune_cache_clear()


def _inputs(lens, seed):
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=seed, io_dtype="bf16", gate_dtype="f32", init_state=True)
    d = device_inputs(inp)
    return inp, d


def _run(d, chunk):
    gdn.timing_start(16)
    o, f = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                       initial_state=d["initial_state"])
    kt = gdn.timing_stop()
    torch.cuda.synchronize()
    return o, f, {k for k, v in kt.items() if v["count"]}


@pytest.mark.parametrize("lens", [[48], [4] * 64, [300] * 8, [4096]], ids=["1x48", "64x4", "8x300", "1x4096"])
def test_tune_picks_fastest_passing_method(lens):
    inp, d = _inputs(lens, seed=gs.SEED_BASE + 700 + len(lens))
    note(f"tune prefill lens={lens[:2]}... n={len(lens)}")
    gdn.tune_cache_clear()
    rule = gdn.method_name(*gdn.prefill_plan(len(lens), sum(lens), 16, 32, 128))
    r = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                         initial_state=d["initial_state"])
    print(f"[tune] n={len(lens)} T={sum(lens)}: rule {rule}, chose {r['method']}; ms {r['ms']}; err {r['err']}",
          flush=True)
    passing = {c: t for c, t in r["ms"].items() if t >= 0}
    assert r["method"] in passing
    assert all(0 <= r["err"][c] <= 1 / 64 for c in passing)
    # the fastest, or the rule's method when none is more than 3% faster
    fastest = min(passing.values())
    if r["method"] == rule:
        assert fastest >= passing[rule] * 0.97
    else:
        assert passing[r["method"]] == fastest and fastest < passing[rule] * 0.97
    assert r["err"]["64/16"] == 0.0  # the reference against itself
    # 32, 64 or 128 state rows per workgroup: the same MFMA sequence per
    # element, the same bits
    for rows in (32, 64, 128):
        assert r["err"][f"64/{rows}"] == 0.0
        assert r["err"][f"32/{rows}"] == r["err"]["32/16"] and r["err"][f"16/{rows}"] == r["err"]["16/16"]
    assert gdn.tune_cache_size() == 1
    # chunk 0 now runs the chosen method: its kernels, its bits
    assert gdn.prefill_plan(len(lens), sum(lens), 16, 32, 128) == (r["chunk"], r["rows"])
    o0, f0, ran = _run(d, 0)
    oc, fc, _ = _run(d, r["chunk"])
    assert KERNEL_OF[r["chunk"]] in ran and len({"token_scan", "scan"} & ran) == 1
    assert torch.equal(o0, oc) and torch.equal(f0, fc)
    o_ref, f_ref = oracle_ref(inp)
    assert rel_err(to_f64(o0), o_ref) <= tol("bf16")
    assert rel_err(to_f64(f0), f_ref) <= tol("bf16")


def test_tune_gate_rejects_what_differs():
    """With a zero tolerance only chunk 64 can pass: the reference (16 rows
    per scan workgroup) and 32, 64 and 128 rows, which compute the same bits.
    Every other chunk rounds differently, so it is rejected and never timed."""
    _, d = _inputs([200, 37], seed=gs.SEED_BASE + 710)
    note("tune prefill with gate_tol = 0")
    r = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                         initial_state=d["initial_state"], gate_tol=0.0)
    print(f"[tune] gate 0: chose {r['method']}; ms {r['ms']}; err {r['err']}", flush=True)
    assert r["chunk"] == 64
    for c in ("64/32", "64/64", "64/128"):
        assert r["err"][c] == 0 and r["ms"][c] > 0
    for c in ("32/16", "32/32", "32/64", "32/128", "16/16", "16/32", "16/64", "16/128", "1"):
        assert r["err"][c] > 0 and r["ms"][c] == -1


def test_tune_cache_file_steers_chunk_zero(tmp_path):
    """A saved choice, edited to another method and loaded back, is what
    chunk 0 runs for that shape bucket (and only for it)."""
    _, d = _inputs([20, 10], seed=gs.SEED_BASE + 720)
    note("tune prefill, save, edit, load")
    r = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                         initial_state=d["initial_state"])
    path = tmp_path / "tune.txt"
    gdn.tune_cache_save(str(path))
    fields = path.read_text().split()
    assert len(fields) == 14 and fields[0] == "gdn-tune-v3"
    assert (int(fields[-2]), int(fields[-1])) == (r["chunk"], r["rows"])
    forced = 16 if r["chunk"] != 16 else 32
    path.write_text(" ".join(fields[:-2] + [str(forced), "32"]) + "\n")
    gdn.tune_cache_clear()
    _, _, ran = _run(d, 0)
    assert ran == {"token_scan"}  # T = 30 <= 32: the rule without a choice
    assert gdn.tune_cache_load(str(path)) == 1
    assert gdn.prefill_plan(2, 30, 16, 32, 128) == (forced, 32)
    o0, f0, ran = _run(d, 0)
    oc, fc, _ = _run(d, forced)
    assert "scan" in ran and "token_scan" not in ran
    assert torch.equal(o0, oc) and torch.equal(f0, fc)
    # another bucket (T = 300 rounds to 512, not 64) keeps the rule
    _, d2 = _inputs([150, 150], seed=gs.SEED_BASE + 721)
    _, _, ran = _run(d2, 0)
    assert ran == {"schedule", "prep", "scan"} or ran == {"prep", "scan"}


def test_tuned_choice_keyed_by_evenness():
    """One 2,048-token prompt beside four of 256 (an uneven batch: its longest
    is 3.3 times the mean). The tuner reads the lengths and caches its choice
    as an uneven batch's: a call with the longest length as a hint takes it,
    and so does a call without a hint (the bucket holds no even batch's
    choice). A hint near the mean marks an even batch of the same bucket,
    which has no tuned choice, so that call takes the rule."""
    lens = [2048, 256, 256, 256, 256]
    N, T = len(lens), sum(lens)
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 1720, io_dtype="bf16", gate_dtype="f32")
    d = device_inputs(inp)
    rule = gdn.prefill_plan(N, T, 16, 32, 128)
    note("tune an uneven batch")
    r = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"])
    tuned = (r["chunk"], r["rows"])
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=2048) == tuned
    assert gdn.prefill_plan(N, T, 16, 32, 128) == tuned
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=T // N + 1) == rule
    # the choice is never slower than the hinted rule's method (64/32 here)
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=2048) == tuned
    assert r["ms"][gdn.method_name(*tuned)] <= r["ms"]["64/32"]


def test_even_choice_not_applied_to_a_hinted_uneven_batch():
    """Eight sequences of 512 tokens tuned (an even batch). A hinted uneven
    batch in the same bucket (8 sequences, 2,048 + 7 x 256 tokens) does not
    take that choice but the hinted rule's method; without the hint it
    takes the even batch's choice, as before."""
    lens = [512] * 8
    inp = gs.make_inputs(lens, 16, 32, 128, 128, seed=gs.SEED_BASE + 1730, io_dtype="bf16", gate_dtype="f32")
    d = device_inputs(inp)
    N, T = 8, 2048 + 7 * 256
    hinted_rule = gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=2048)
    note("tune an even batch")
    r = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"])
    tuned = (r["chunk"], r["rows"])
    assert gdn.prefill_plan(N, T, 16, 32, 128, max_seqlen=2048) == hinted_rule
    assert gdn.prefill_plan(N, T, 16, 32, 128) == tuned
