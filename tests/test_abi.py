"""The C ABI on the host: symbols, sizes and argument checks (no GPU needed).

Every call here is rejected by host-side validation before any HIP call is
made, so it runs on machines without a GPU. Fake device pointers are plain
non-zero integers; the library never dereferences them on the host.
"""

import ctypes
import os
import re

import pytest
import torch

import gated_deltanet_linear_02_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE, HIP, ALIAS, BAD_VALUE, MISALIGNED = range(9)
BF16, F32 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.lib_path()):
        from gated_deltanet_linear_02_amd import build
        build.build()
    return gdn.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"gdn_prefill", "gdn_decode_step", "gdn_prefill_workspace_size",
            "gdn_prefill_ex", "gdn_decode_step_ex", "gdn_tune_prefill", "gdn_tune_cache_load",
            "gdn_status_string", "gdn_abi_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gdn.h but not exported"


def test_version_and_status_strings(lib):
    assert gdn.abi_version() == 5
    for s in range(9):
        assert lib.gdn_status_string(s)
    assert b"unknown" in lib.gdn_status_string(99)


def _ws(n=1, T=4096, hk=16, hv=32, d=128, c=64, io=BF16):
    return gdn.load().gdn_prefill_workspace_size(n, T, hk, hv, d, d, c, io)


def test_workspace_size(lib):
    w = _ws()
    # per chunk: Tb and P (bf16 C x C) and W (bf16 C x d) per value head, Q
    # and K^T per query/key head (bf16 C x d), and per value head a gate
    # record of 2C + 4 fp32 (delta and scale*gamma per token, gamma_C, padding)
    # and d/16 slots of C fp32 for the fused normalisation's partial sums
    # chunks: at most floor((T + N (C - 1)) / C) over N sequences, which
    # for one sequence is ceil(T / C)
    chunks = (4096 + 63) // 64
    need = chunks * (32 * (2 * 64 * 64 * 2 + 64 * 128 * 2 + (2 * 64 + 4) * 4 + (128 // 16) * 64 * 4)
                     + 16 * 2 * 64 * 128 * 2)
    assert need <= w < need + 64 * 1024
    assert _ws(io=F32) > w
    assert _ws(T=0) > 0
    # rejected shapes give 0
    assert _ws(hk=3, hv=32) == 0
    assert _ws(d=96) == 0
    assert _ws(c=48) == 0
    assert _ws(n=0) == 0
    # token by token (chunk 1) needs no workspace; a nonzero size still means
    # "accepted".
    assert _ws(c=1) == 256 and _ws(c=1, T=1 << 20) == 256
    # chunk 0 may take a tuned choice, so it covers every chunked method
    for n, T in ((1, 64), (64, 1024), (1, 65), (1, 4096), (8, 2400)):
        assert _ws(c=0, n=n, T=T) == max(_ws(c=c, n=n, T=T) for c in (16, 32, 64)) > 256
    assert _ws(c=2) == 0 and _ws(c=-1) == 0


FAKE = 0x7F0000000000

# The checks below pass fake device pointers and expect host-side rejection.
# On a machine with a GPU a validation bug would launch a kernel on them, so
# they only run where no GPU is visible.
no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake-pointer validation tests run only on hosts without a GPU")


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), cu=FAKE + (5 << 30), n=1, T=128, hk=2, hv=4, dk=64, dv=64,
             chunk=64, scale=1.0, io=BF16, gate=F32, s0=None, sf=None, out=FAKE + (6 << 30),
             ws=FAKE + (7 << 30), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
                           a["hk"], a["hv"], a["dk"], a["dv"], a["chunk"], a["scale"], a["io"],
                           a["gate"], a["s0"], a["sf"], a["out"], a["ws"], a["ws_bytes"], a["stream"])


@no_gpu
def test_prefill_argument_checks(lib):
    assert _prefill(lib, q=None) == NULL_ARG
    assert _prefill(lib, cu=None) == NULL_ARG
    assert _prefill(lib, out=None) == NULL_ARG
    assert _prefill(lib, hk=3, hv=4) == BAD_SHAPE
    assert _prefill(lib, n=0) == BAD_SHAPE
    assert _prefill(lib, T=-1) == BAD_SHAPE
    assert _prefill(lib, T=1 << 33) == BAD_SHAPE
    assert _prefill(lib, dk=96, dv=96) == UNSUPPORTED
    assert _prefill(lib, dk=64, dv=128) == UNSUPPORTED
    assert _prefill(lib, chunk=128) == UNSUPPORTED
    assert _prefill(lib, chunk=8) == UNSUPPORTED
    assert _prefill(lib, chunk=-1) == UNSUPPORTED
    assert _prefill(lib, io=7) == UNSUPPORTED
    assert _prefill(lib, gate=2) == UNSUPPORTED
    assert _prefill(lib, ws=None) == WORKSPACE
    assert _prefill(lib, ws_bytes=100) == WORKSPACE
    assert _prefill(lib, ws=FAKE + (7 << 30) + 16) == WORKSPACE  # misaligned
    # out overlapping an input
    assert _prefill(lib, out=FAKE + 64) == ALIAS
    assert _prefill(lib, out=FAKE + (4 << 30) + 16) == ALIAS
    # final state overlapping q
    assert _prefill(lib, sf=FAKE + 128) == ALIAS
    # the workspace overlapping an input: q, v, cu_seqlens, the initial state
    assert _prefill(lib, ws=FAKE + 256) == ALIAS
    assert _prefill(lib, ws=FAKE + (2 << 30) - 256) == ALIAS
    assert _prefill(lib, ws=FAKE + (5 << 30)) == ALIAS
    assert _prefill(lib, s0=FAKE + (8 << 30), ws=FAKE + (8 << 30) + 4096) == ALIAS
    # tensors read in 16-byte pieces must be 16-byte aligned (gates need not)
    assert _prefill(lib, q=FAKE + 8) == MISALIGNED
    assert _prefill(lib, out=FAKE + (6 << 30) + 2) == MISALIGNED
    assert _prefill(lib, s0=FAKE + (8 << 30) + 4) == MISALIGNED
    assert _prefill(lib, g=FAKE + (3 << 30) + 4, beta=FAKE + (4 << 30) + 4) != MISALIGNED
    # in-place final == initial state is allowed by validation (it would launch
    # next, so it is not called here); overlapping but different is not
    assert _prefill(lib, s0=FAKE + (8 << 30), sf=FAKE + (8 << 30) + 16) == ALIAS


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), B=64, hk=16, hv=32, dk=128, dv=128, scale=1.0, io=BF16,
             gate=BF16, state=FAKE + (5 << 30), slots=None, num_slots=64,
             out=FAKE + (9 << 30), stream=None)
    a.update(kw)
    return lib.gdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["B"], a["hk"], a["hv"],
                               a["dk"], a["dv"], a["scale"], a["io"], a["gate"], a["state"],
                               a["slots"], a["num_slots"], a["out"], a["stream"])


@no_gpu
def test_decode_argument_checks(lib):
    assert _decode(lib, B=0) == OK  # nothing to do, nothing launched
    assert _decode(lib, state=None) == NULL_ARG
    assert _decode(lib, v=None) == NULL_ARG
    assert _decode(lib, B=-1) == BAD_SHAPE
    assert _decode(lib, hk=5) == BAD_SHAPE
    assert _decode(lib, num_slots=10) == BAD_SHAPE  # identity slots need num_slots >= batch
    assert _decode(lib, dk=48, dv=48) == UNSUPPORTED
    assert _decode(lib, io=3) == UNSUPPORTED
    assert _decode(lib, out=FAKE + 96) == ALIAS
    assert _decode(lib, out=FAKE + (5 << 30) + 4096) == ALIAS  # out inside the state
    assert _decode(lib, state=FAKE + (2 << 30) + 64) == ALIAS  # state over v
    assert _decode(lib, v=FAKE + (2 << 30) + 2) == MISALIGNED
    assert _decode(lib, state=FAKE + (5 << 30) + 4) == MISALIGNED


def test_timing_stop_without_start(lib):
    assert lib.gdn_timing_stop(None, None, 0) == BAD_SHAPE
    assert lib.gdn_timing_start(0) == BAD_SHAPE


def test_binding_raises_on_missing_library(tmp_path, monkeypatch):
    import importlib
    mod = importlib.reload(gdn)
    monkeypatch.setattr(mod, "_LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        mod.load()
    importlib.reload(gdn)


NORM_W = FAKE + (10 << 30)


def _prefill_ex(lib, w=NORM_W, eps=1e-6, sdt=F32, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), cu=FAKE + (5 << 30), n=1, T=128, hk=2, hv=4, dk=64, dv=64,
             chunk=64, scale=1.0, io=BF16, gate=F32, s0=None, sf=None, out=FAKE + (6 << 30),
             ws=FAKE + (7 << 30), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.gdn_prefill_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
                              a["hk"], a["hv"], a["dk"], a["dv"], a["chunk"], a["scale"], a["io"],
                              a["gate"], a["s0"], a["sf"], sdt, w, eps, a["out"], a["ws"], a["ws_bytes"],
                              a["stream"])


def _decode_ex(lib, w=NORM_W, eps=1e-6, sdt=F32, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), B=64, hk=16, hv=32, dk=128, dv=128, scale=1.0, io=BF16,
             gate=BF16, state=FAKE + (5 << 30), slots=None, num_slots=64,
             out=FAKE + (9 << 30), stream=None)
    a.update(kw)
    return lib.gdn_decode_step_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["B"], a["hk"],
                                  a["hv"], a["dk"], a["dv"], a["scale"], a["io"], a["gate"],
                                  a["state"], sdt, a["slots"], a["num_slots"], w, eps, a["out"],
                                  a["stream"])


@no_gpu
def test_ex_argument_checks(lib):
    inf, nan = float("inf"), float("nan")
    for call in (_prefill_ex, _decode_ex):
        assert call(lib, eps=-1e-6) == BAD_VALUE
        assert call(lib, eps=inf) == BAD_VALUE
        assert call(lib, eps=nan) == BAD_VALUE
        # the weight is an input: out must not overlap it
        assert call(lib, w=FAKE + (6 << 30) + 64 if call is _prefill_ex else FAKE + (9 << 30) + 64) == ALIAS
        # the other checks are those of the plain entry points
        assert call(lib, hk=3) == BAD_SHAPE
        assert call(lib, dk=96, dv=96) == UNSUPPORTED
        # state storage: fp32 or bf16, and bf16 only with bf16 I/O
        assert call(lib, sdt=2) == UNSUPPORTED
        assert call(lib, sdt=BF16, io=F32) == UNSUPPORTED
        assert call(lib, sdt=BF16, w=None, io=F32) == UNSUPPORTED
    # decode: the state is written, so it must not overlap the weight
    assert _decode_ex(lib, w=FAKE + (5 << 30) + 4096) == ALIAS
    # the state's extent follows its dtype: a bf16 pool of 64 slots is half
    # as long, so an output just past it is fine for bf16 and overlaps fp32
    past_bf16 = FAKE + (5 << 30) + 64 * 32 * 128 * 128 * 2
    assert _decode_ex(lib, out=past_bf16, sdt=F32) == ALIAS
    # prefill: the final state must not overlap the weight either
    assert _prefill_ex(lib, sf=NORM_W - 64) == ALIAS
    assert _prefill_ex(lib, ws=None) == WORKSPACE
    assert _decode_ex(lib, B=0) == OK


def _prefill_hint(lib, hint, w=NORM_W, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), cu=FAKE + (5 << 30), n=3, T=382, hk=2, hv=4, dk=64, dv=64,
             chunk=0, scale=1.0, io=BF16, gate=F32, s0=None, sf=None, out=FAKE + (6 << 30),
             ws=FAKE + (7 << 30), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.gdn_prefill_hint(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"], hint,
                                a["hk"], a["hv"], a["dk"], a["dv"], a["chunk"], a["scale"], a["io"],
                                a["gate"], a["s0"], a["sf"], F32, w, 1e-6, a["out"], a["ws"], a["ws_bytes"],
                                a["stream"])


@no_gpu
def test_prefill_hint_argument_checks(lib):
    """A max_seqlen hint lies between the mean length and the total; the
    other checks are those of gdn_prefill_ex, made before the hint's."""
    assert _prefill_hint(lib, 127) == BAD_VALUE   # below the mean of 382 / 3
    assert _prefill_hint(lib, 383) == BAD_VALUE   # above the total
    assert _prefill_hint(lib, -1) == BAD_VALUE
    assert _prefill_hint(lib, 300, hk=3) == BAD_SHAPE
    assert _prefill_hint(lib, 300, w=FAKE + (6 << 30) + 64) == ALIAS
    assert _prefill_hint(lib, 300, ws=None) == WORKSPACE
    assert _prefill_hint(lib, 0, ws=None) == WORKSPACE


def test_max_seqlen_hint_plans():
    """With the longest length as a hint, uneven batches take the state rows
    (and for short ones the chunk) that the tuner measures fastest; even
    batches, or a hint within 1.25 times the mean, keep the rule's method."""
    def p(lens, **kw):
        return gdn.prefill_plan(len(lens), sum(lens), 16, 32, 128, **kw)
    varlen = [1541, 2796, 5227, 7117, 8976, 10781, 12892, 14620]
    assert p(varlen) == (64, 128) and p(varlen, max_seqlen=14620) == (64, 64)
    assert p([4096] + [512] * 4) == (64, 128) and p([4096] + [512] * 4, max_seqlen=4096) == (64, 32)
    assert p([8192, 1024, 1024], max_seqlen=8192) == (64, 16)
    assert p([2048, 1024, 512, 256], max_seqlen=2048) == (64, 32)
    assert p([300, 77, 5], max_seqlen=300) == (32, 32)
    for lens in ([1024] * 8, [512] * 8, [2048] * 2, [200] * 3, [4096], [600, 500, 400], [128] * 32):
        assert p(lens, max_seqlen=max(lens)) == p(lens), lens
    # other head layouts: the longest length decides the chunk (HK 8, HV 16,
    # d 64: one pass, but a 2,048-token chain)
    assert gdn.prefill_plan(4, 3840, 8, 16, 64) == (32, 16)
    assert gdn.prefill_plan(4, 3840, 8, 16, 64, max_seqlen=2048) == (64, 16)
    # many tiny sequences beside a longer one: chunked once the longest
    # exceeds 16 + 2 N tokens, with chunks by the longest length
    assert p([500] + [1] * 63) == (1, 0) and p([500] + [1] * 63, max_seqlen=500) == (32, 128)
    assert p([120] + [3] * 20, max_seqlen=120) == (16, 128)
    assert p([64] + [1] * 63, max_seqlen=64) == (1, 0)
    assert p([1000] + [2] * 100, max_seqlen=1000) == (32, 128)
    # fp32 I/O: 16-row slices whatever the hint; short uneven batches take
    # chunks of 32, and tiny means stay token by token
    f32 = torch.float32
    assert p(varlen, io_dtype=f32, max_seqlen=14620) == (64, 16)
    assert p([300, 77, 5], io_dtype=f32) == (64, 16) and p([300, 77, 5], io_dtype=f32, max_seqlen=300) == (32, 16)
    assert p([500] + [1] * 63, io_dtype=f32, max_seqlen=500) == (1, 0)
    # hints outside [mean, total] are refused
    assert p([300, 77, 5], max_seqlen=100) == (0, 0) and p([300, 77, 5], max_seqlen=383) == (0, 0)


def test_tune_cache_file_round_trip(tmp_path):
    """The tuning cache's text file: well-formed lines (evenness, then chunk
    and state rows per scan workgroup, 16 to 128) load; malformed ones,
    unknown methods and other formats are skipped; and a save writes what
    was loaded."""
    lib = gdn.load()
    gdn.tune_cache_clear()
    src = tmp_path / "tune.txt"
    src.write_text(
        "gdn-tune-v3 gfx950/256cu 70000 5002 1 4096 16 32 128 0 1 0 64 16\n"
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 65536 16 32 128 0 1 0 64 128\n"
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 65536 16 32 128 0 1 1 64 64\n"  # the same bucket, uneven
        "gdn-tune-v3 gfx950/256cu 70000 5002 4 4096 16 32 128 0 1 0 64 32\n"
        "gdn-tune-v3 gfx950/256cu 70000 5002 64 1024 16 32 128 0 0 0 1 0\n"
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 512 2 4 64 1 1 0 48 16\n"  # not a chunk
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 512 2 4 64 1 1 0 64 8\n"   # not a row count
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 512 2 4 64 1 1 0 1 16\n"   # token by token has no rows
        "gdn-tune-v3 gfx950/256cu 70000 5002 8 512 2 4 64 1 1 2 64 16\n"  # evenness is 0 or 1
        "gdn-tune-v2 gfx950/256cu 70000 4002 8 512 2 4 64 1 1 64 16\n"    # older format
        "garbage\n")
    assert gdn.tune_cache_load(str(src)) == 5
    assert gdn.tune_cache_size() == 5
    out = tmp_path / "saved.txt"
    gdn.tune_cache_save(str(out))
    lines = sorted(out.read_text().splitlines())
    assert lines == sorted(src.read_text().splitlines()[:5])
    gdn.tune_cache_clear()
    assert gdn.tune_cache_size() == 0
    with pytest.raises(gdn.GdnError):
        gdn.tune_cache_load(str(tmp_path / "missing.txt"))
    assert lib.gdn_tune_cache_save(None) == NULL_ARG


def test_tune_scratch_size(lib):
    size = lib.gdn_tune_prefill_scratch_size(1, 4096, 16, 32, 128, 128, BF16)
    out_b = 4096 * 32 * 128 * 2
    fin_b = 32 * 128 * 128 * 4
    assert size >= 2 * out_b + 2 * fin_b + _ws(c=0)
    assert lib.gdn_tune_prefill_scratch_size(1, 4096, 3, 32, 128, 128, BF16) == 0


@no_gpu
def test_tune_argument_checks(lib):
    chosen = ctypes.c_int32(0)
    # host-side rejections (nothing is launched)
    args = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30),
            1, 128, 2, 4, 64, 64, 1.0, BF16, F32, None]
    need = lib.gdn_tune_prefill_scratch_size(1, 128, 2, 4, 64, 64, BF16)
    assert lib.gdn_tune_prefill(*args, 1.0 / 64, FAKE + (6 << 30), need, None, None, None, None, None) == NULL_ARG
    assert lib.gdn_tune_prefill(*args, -0.1, FAKE + (6 << 30), need, None, ctypes.byref(chosen), None, None,
                                None) == BAD_VALUE
    assert lib.gdn_tune_prefill(*args, 1.0 / 64, FAKE + (6 << 30), need - 1, None, ctypes.byref(chosen), None,
                                None, None) == WORKSPACE
    assert lib.gdn_tune_prefill(*args, 1.0 / 64, None, need, None, ctypes.byref(chosen), None, None,
                                None) == WORKSPACE


def test_chunk_zero_rule(lib):
    """The method chunk 0 takes with nothing tuned, by mean sequence length
    (HK=16, HV=32, d=128, bf16; the scan fills the GPU in one pass up to one
    sequence with 16-row slices, two with 32-row, four with 64-row and eight
    with 128-row slices)."""
    gdn.tune_cache_clear()
    m = lambda n, T: gdn.prefill_method(n, T, 16, 32, 128)
    assert m(1, 16) == 1 and m(1, 32) == 1          # one short prompt
    assert m(64, 64 * 10) == 1 and m(8, 8 * 4) == 1  # batches, mean <= 10
    assert m(1, 48) == 16 and m(2, 2 * 48) == 16     # 16- or 32-row slices, mean <= 48
    assert m(64, 64 * 16) == 16 and m(64, 64 * 24) == 32 and m(64, 64 * 33) == 64  # 128-row slices
    assert m(1, 128) == 32 and m(1, 1024) == 32      # one sequence: one pass
    assert m(1, 4096) == 64 and m(8, 8 * 300) == 64  # long, or several passes
    assert m(2, 2 * 600) == 32                       # two sequences: one pass of 32-row slices
    assert m(4, 4 * 600) == 64                       # four: 64-row slices, whose long step wants chunks of 64
    # fp32 I/O: token by token up to L = 48, chunks of 32 for one pass and L <= 512, else 64
    f32 = lambda n, T: gdn.prefill_method(n, T, 16, 32, 128, io_dtype=torch.float32)
    assert f32(1, 16) == 1 and f32(64, 64 * 48) == 1 and f32(64, 64 * 49) == 64
    assert f32(1, 128) == 32 and f32(1, 512) == 32 and f32(1, 1024) == 64 and f32(1, 4096) == 64
    assert f32(2, 2 * 600) == 64 and f32(8, 8 * 300) == 64
    assert gdn.prefill_method(1, 4096, 16, 32, 128, chunk=16) == 16  # explicit chunks as given
    assert gdn.prefill_method(1, 4096, 3, 32, 128) == 0              # rejected shape
    # state rows per scan workgroup: the fewest of 16, 32, 64, 128 whose
    # N * HV * DV / rows workgroups fit 256 CUs in one pass, else the most;
    # more than 16 for bf16 I/O only, and at most d
    p = lambda n, T, hv=32, d=128, io=torch.bfloat16, c=0: gdn.prefill_plan(n, T, 16, hv, d, c, io)
    assert p(1, 4096) == (64, 16) and p(2, 2 * 4096) == (64, 32)
    assert p(4, 4 * 1024) == (64, 64) and p(8, 8 * 512) == (64, 128)
    assert p(32, 32 * 128) == (64, 128)                              # 1024 workgroups even so
    assert p(64, 64 * 16) == (16, 128) and p(64, 64 * 32) == (32, 128)  # one chunk per sequence
    assert p(8, 8 * 512, d=64) == (64, 64) and p(8, 8 * 512, d=32) == (32, 32)  # at most d
    assert p(1, 4096, hv=48) == (64, 32)                             # 384 slices of 16 rows
    assert p(2, 2 * 4096, io=torch.float32) == (64, 16)              # fp32 I/O: 16 rows
    assert p(64, 64 * 4, c=1) == (1, 0) and p(64, 64 * 4) == (1, 0)  # token by token: no scan
    assert p(40, 40 * 100, d=16, hv=16) == (64, 16)                  # d = 16: 16 rows
    assert p(1, 4096, hv=3) == (0, 0)                                 # rejected


def test_binding_checks_shapes_before_calling():
    """The binding refuses tensors that do not match the call's sizes (the
    library would access them past their ends); CPU tensors suffice, since
    the checks run before anything reaches the library."""
    import torch
    T, hk, hv, d = 8, 2, 4, 16
    q = torch.zeros((T, hk, d), dtype=torch.bfloat16)
    ok = dict(k=torch.zeros((T, hk, d), dtype=torch.bfloat16), v=torch.zeros((T, hv, d), dtype=torch.bfloat16),
              g=torch.zeros((T, hv)), beta=torch.zeros((T, hv)))
    cu = torch.tensor([0, T], dtype=torch.int32)
    bad = [dict(v=torch.zeros((T - 1, hv, d), dtype=torch.bfloat16)),
           dict(k=torch.zeros((T, hk, d), dtype=torch.float32)),
           dict(beta=torch.zeros((T, hv + 1))),
           dict(beta=torch.zeros((T, hv), dtype=torch.bfloat16))]
    for b in bad:
        a = {**ok, **b}
        with pytest.raises((ValueError, TypeError)):
            gdn.prefill(q, a["k"], a["v"], a["g"], a["beta"], cu)
    with pytest.raises(ValueError):
        gdn.prefill(q, ok["k"], ok["v"], ok["g"], ok["beta"], cu,
                    initial_state=torch.zeros((2, hv, d, d)))
    with pytest.raises(ValueError):
        gdn.decode_step(q, ok["k"], ok["v"][:4], ok["g"], ok["beta"], torch.zeros((T, hv, d, d)))


@no_gpu
def test_prefill_noalloc_host_checks(lib):
    """The fixed-workspace entry point rejects, before any HIP call, shapes
    the other entry points reject and a method whose workspace exceeds the
    array (T = 32768 at chunk 64)."""
    vp = ctypes.c_void_p

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
                 beta=FAKE + (4 << 30), cu=FAKE + (5 << 30), n=1, T=32768, hk=16, hv=32, dk=128, dv=128,
                 chunk=64, scale=1.0, io=BF16, gate=F32, s0=None, sf=None, out=FAKE + (6 << 30), stream=None)
        a.update(kw)
        return lib.gdn_prefill_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
                                       a["hk"], a["hv"], a["dk"], a["dv"], a["chunk"], a["scale"], a["io"],
                                       a["gate"], a["s0"], a["sf"], a["out"], a["stream"])
    assert call() == WORKSPACE
    assert call(hk=3, hv=4) == BAD_SHAPE
    assert call(dk=96, dv=96) == UNSUPPORTED
    assert call(chunk=8) == UNSUPPORTED
    # the largest single bf16 sequence that fits at chunk 64 (5,184 tokens,
    # 81 chunks) and the next one
    assert lib.gdn_prefill_workspace_size(1, 5184, 16, 32, 128, 128, 64, BF16) <= 128 << 20
    assert lib.gdn_prefill_workspace_size(1, 5185, 16, 32, 128, 128, 64, BF16) > 128 << 20
    assert call(T=5185) == WORKSPACE
