"""Pins for the CPU oracle, against facts that do not come from the oracle.

Each test fixes one part of the gated delta rule
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = scale S_t q_t,
so that a dropped term, a wrong sign, a transposed state or a wrong head
mapping in the oracle fails at least one of them:

  closed forms      b = 0 (decay only), a -> 0 (reset), hand-worked values
  invariants        retrieval with b = 1 and unit keys, linearity in (S0, V),
                    split/varlen/permutation invariance, head sharing
  cross-form        explicit-matrix recurrence and chunk-parallel (WY) form
                    agree with the token loop on tiny inputs
"""

import json
import os

import numpy as np
import pytest

import gdn_synth as gs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, seqlens, hk, hv, d, unit_k=True):
    T = int(sum(seqlens))
    q = rng.standard_normal((T, hk, d))
    k = rng.standard_normal((T, hk, d))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, hv, d))
    g = -np.log1p(np.exp(rng.normal(-1.0, 1.0, (T, hv))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, hv))))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return q, k, v, g, b, cu


def _rel(a, b):
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


# ---------------------------------------------------------------- closed forms

def test_hand_worked_golden():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        toks = case["tokens"]
        T = len(toks)
        d_k, d_v = case["dk"], case["dv"]
        q = np.array([t["q"] for t in toks], dtype=np.float64).reshape(T, 1, d_k)
        k = np.array([t["k"] for t in toks], dtype=np.float64).reshape(T, 1, d_k)
        v = np.array([t["v"] for t in toks], dtype=np.float64).reshape(T, 1, d_v)
        g = np.log(np.array([t["a"] for t in toks], dtype=np.float64)).reshape(T, 1)
        b = np.array([t["b"] for t in toks], dtype=np.float64).reshape(T, 1)
        s0 = np.array(case["s0"], dtype=np.float64).reshape(1, 1, d_v, d_k)
        cu = np.array([0, T])
        out, fin = oracle.scan(q, k, v, g, b, cu, scale=case["scale"], initial_state=s0)
        np.testing.assert_allclose(out.reshape(T, d_v), np.array(case["expect_out"]),
                                   rtol=1e-15, atol=1e-15, err_msg=case["name"])
        np.testing.assert_allclose(fin.reshape(d_v, d_k), np.array(case["expect_state"]),
                                   rtol=1e-15, atol=1e-15, err_msg=case["name"])
        out2, fin2 = oracle.literal_scan(q, k, v, g, b, cu, scale=case["scale"], initial_state=s0)
        np.testing.assert_allclose(out2.reshape(T, d_v), np.array(case["expect_out"]),
                                   rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(fin2.reshape(d_v, d_k), np.array(case["expect_state"]),
                                   rtol=1e-15, atol=1e-15)


def test_no_write_no_decay_keeps_state():
    """b = 0, a = 1: S_t = S_0 and o_t = scale S_0 q_t."""
    rng = np.random.default_rng(1)
    q, k, v, g, b, cu = _rand_inputs(rng, [37], 2, 4, 16)
    g[:] = 0.0
    b[:] = 0.0
    s0 = rng.standard_normal((1, 4, 16, 16))
    out, fin = oracle.scan(q, k, v, g, b, cu, scale=0.75, initial_state=s0)
    np.testing.assert_allclose(fin, s0, rtol=0, atol=0)
    for h in range(4):
        expect = 0.75 * q[:, h // 2] @ s0[0, h].T
        np.testing.assert_allclose(out[:, h], expect, rtol=1e-14, atol=1e-14)


def test_decay_only_closed_form():
    """b = 0: S_t = exp(sum_{s<=t} g_s) S_0, o_t = scale exp(c_t) S_0 q_t."""
    rng = np.random.default_rng(2)
    q, k, v, g, b, cu = _rand_inputs(rng, [50], 2, 2, 8)
    b[:] = 0.0
    s0 = rng.standard_normal((1, 2, 8, 8))
    out, fin = oracle.scan(q, k, v, g, b, cu, initial_state=s0)
    for h in range(2):
        c = np.cumsum(g[:, h])
        np.testing.assert_allclose(fin[0, h], np.exp(c[-1]) * s0[0, h], rtol=1e-13)
        expect = np.exp(c)[:, None] * (q[:, h // 1] @ s0[0, h].T)
        np.testing.assert_allclose(out[:, h], expect, rtol=1e-12, atol=1e-15)


def test_reset_when_decay_underflows():
    """a = exp(-1e4) = 0 in double: S_t = b_t v_t k_t^T, o_t = b_t (k_t.q_t) v_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, b, cu = _rand_inputs(rng, [20], 1, 1, 8, unit_k=False)
    g[:] = -1.0e4
    s0 = rng.standard_normal((1, 1, 8, 8))
    out, fin = oracle.scan(q, k, v, g, b, cu, initial_state=s0)
    t = 19
    np.testing.assert_allclose(fin[0, 0], b[t, 0] * np.outer(v[t, 0], k[t, 0]), rtol=1e-14)
    expect = (b[:, 0] * np.sum(k[:, 0] * q[:, 0], axis=-1))[:, None] * v[:, 0]
    np.testing.assert_allclose(out[:, 0], expect, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_full_write_retrieves_value():
    """b = 1 and |k| = 1: S_t k_t = v_t exactly, for any decay and any prior state."""
    rng = np.random.default_rng(4)
    for T in (1, 2, 9):
        q, k, v, g, b, cu = _rand_inputs(rng, [T], 2, 2, 16)
        b[:] = 1.0
        s0 = rng.standard_normal((1, 2, 16, 16))
        # final state after the last token must map k_T to v_T
        _, fin = oracle.scan(q, k, v, g, b, cu, initial_state=s0)
        for h in range(2):
            np.testing.assert_allclose(fin[0, h] @ k[-1, h], v[-1, h], rtol=1e-12, atol=1e-12)
        # and a query equal to the key reads the value back in the output
        q2 = k.copy()
        out, _ = oracle.scan(q2, k, v, g, b, cu, initial_state=s0)
        np.testing.assert_allclose(out, v, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_store_all_values():
    """a = 1, b = 1, orthonormal keys, S_0 = 0: S_n k_i = v_i for every i <= n."""
    rng = np.random.default_rng(5)
    d = 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[:12].reshape(12, 1, d)  # 12 orthonormal rows
    v = rng.standard_normal((12, 1, d))
    q = k.copy()
    g = np.zeros((12, 1))
    b = np.ones((12, 1))
    out, fin = oracle.scan(q, k, v, g, b, np.array([0, 12]))
    S = fin[0, 0]
    for i in range(12):
        np.testing.assert_allclose(S @ k[i, 0], v[i, 0], rtol=1e-12, atol=1e-12)
    # standard-basis keys in the loop too
    e = np.eye(d)[:5].reshape(5, 1, d)
    v5 = rng.standard_normal((5, 1, d))
    _, fin5 = oracle.scan(e, e, v5, np.zeros((5, 1)), np.ones((5, 1)), np.array([0, 5]))
    np.testing.assert_allclose(fin5[0, 0][:, :5], v5[:, 0].T, rtol=0, atol=0)
    np.testing.assert_allclose(fin5[0, 0][:, 5:], 0.0, rtol=0, atol=0)


def test_linear_in_state_and_values():
    """For fixed q, k, g, b the map (S_0, V) -> (O, S_T) is linear."""
    rng = np.random.default_rng(6)
    q, k, v1, g, b, cu = _rand_inputs(rng, [31], 2, 4, 16)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, 4, 16, 16))
    s2 = rng.standard_normal((1, 4, 16, 16))
    al, be = 0.7, -1.3
    o1, f1 = oracle.scan(q, k, v1, g, b, cu, initial_state=s1)
    o2, f2 = oracle.scan(q, k, v2, g, b, cu, initial_state=s2)
    o3, f3 = oracle.scan(q, k, al * v1 + be * v2, g, b, cu, initial_state=al * s1 + be * s2)
    assert _rel(o3, al * o1 + be * o2) < 1e-12
    assert _rel(f3, al * f1 + be * f2) < 1e-12
    # and the output is linear in scale
    o4, _ = oracle.scan(q, k, v1, g, b, cu, initial_state=s1, scale=-2.5)
    assert _rel(o4, -2.5 * o1) < 1e-15


def test_split_invariance():
    """Prefill [0, T) equals [0, m) then [m, T) with the final state carried."""
    rng = np.random.default_rng(7)
    q, k, v, g, b, cu = _rand_inputs(rng, [45], 2, 4, 16)
    s0 = rng.standard_normal((1, 4, 16, 16))
    o, f = oracle.scan(q, k, v, g, b, cu, initial_state=s0)
    for m in (0, 1, 17, 44, 45):
        oa, fa = oracle.scan(q[:m], k[:m], v[:m], g[:m], b[:m], np.array([0, m]), initial_state=s0)
        ob, fb = oracle.scan(q[m:], k[m:], v[m:], g[m:], b[m:], np.array([0, 45 - m]), initial_state=fa)
        np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=0)
        np.testing.assert_allclose(fb, f, rtol=0, atol=0)


def test_varlen_equals_separate_and_permutes():
    rng = np.random.default_rng(8)
    lens = [5, 0, 23, 1, 12]
    q, k, v, g, b, cu = _rand_inputs(rng, lens, 2, 4, 8)
    s0 = rng.standard_normal((len(lens), 4, 8, 8))
    o, f = oracle.scan(q, k, v, g, b, cu, initial_state=s0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, fn = oracle.scan(q[sl], k[sl], v[sl], g[sl], b[sl], np.array([0, lens[n]]),
                             initial_state=s0[n:n + 1])
        np.testing.assert_allclose(o[sl], on, rtol=0, atol=0)
        np.testing.assert_allclose(f[n], fn[0], rtol=0, atol=0)
    # empty sequence: final state is the initial state
    np.testing.assert_allclose(f[1], s0[1], rtol=0, atol=0)
    # permuting sequences permutes results
    perm = [3, 0, 4, 2, 1]
    parts = [(slice(cu[n], cu[n + 1])) for n in perm]
    cat = lambda x: np.concatenate([x[p] for p in parts])
    cu_p = np.concatenate([[0], np.cumsum([lens[n] for n in perm])])
    op, fp = oracle.scan(cat(q), cat(k), cat(v), cat(g), cat(b), cu_p, initial_state=s0[perm])
    np.testing.assert_allclose(op, cat(o), rtol=0, atol=0)
    np.testing.assert_allclose(fp, f[perm], rtol=0, atol=0)


def test_head_sharing_equals_duplicated_heads():
    """hk = 2 shared by hv = 4 equals hk = hv = 4 with q/k head h//2 copied."""
    rng = np.random.default_rng(9)
    q, k, v, g, b, cu = _rand_inputs(rng, [19], 2, 4, 8)
    o, f = oracle.scan(q, k, v, g, b, cu)
    qd = np.repeat(q, 2, axis=1)
    kd = np.repeat(k, 2, axis=1)
    o2, f2 = oracle.scan(qd, kd, v, g, b, cu)
    np.testing.assert_allclose(o, o2, rtol=0, atol=0)
    np.testing.assert_allclose(f, f2, rtol=0, atol=0)
    # and heads=subset computes exactly those heads
    o3, f3 = oracle.scan(q, k, v, g, b, cu, heads=[3, 1])
    np.testing.assert_allclose(o3[:, [1, 3]], o[:, [1, 3]], rtol=0, atol=0)
    assert np.all(o3[:, [0, 2]] == 0)


def test_threads_do_not_change_bits():
    inp = gs.workload("tiny")
    w = inp.widened()
    args = [w[x] for x in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    o1, f1 = oracle.scan(*args, threads=1)
    o2, f2 = oracle.scan(*args, threads=7)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_decode_step_is_one_token_scan():
    rng = np.random.default_rng(10)
    q, k, v, g, b, _ = _rand_inputs(rng, [6], 2, 4, 8)
    s = rng.standard_normal((6, 4, 8, 8))
    o, f = oracle.decode_step(q, k, v, g, b, s)
    for n in range(6):
        on, fn = oracle.literal_scan(q[n:n + 1], k[n:n + 1], v[n:n + 1], g[n:n + 1], b[n:n + 1],
                                     np.array([0, 1]), initial_state=s[n:n + 1])
        assert _rel(o[n], on[0]) < 1e-14
        assert _rel(f[n], fn[0]) < 1e-14


# ---------------------------------------------------------------- cross-form

@pytest.mark.parametrize("chunk", [1, 2, 7, 16, 64])
def test_chunked_form_equals_scan(chunk):
    """The chunk-parallel (WY) form equals the token loop, partial chunks included."""
    inp = gs.workload("tiny")
    w = inp.widened()
    rng = np.random.default_rng(11)
    s0 = rng.standard_normal((1, 2, 16, 16)) * 0.02
    args = [w[x] for x in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    o, f = oracle.scan(*args, initial_state=s0)
    oc, fc = oracle.chunked(*args, chunk=chunk, initial_state=s0)
    assert _rel(oc, o) < 1e-12
    assert _rel(fc, f) < 1e-12
    # varlen with ragged tails
    q, k, v, g, b, cu = _rand_inputs(rng, [7, 30, 1, 18], 1, 2, 8)
    s1 = rng.standard_normal((4, 2, 8, 8))
    o, f = oracle.scan(q, k, v, g, b, cu, initial_state=s1, scale=0.5)
    oc, fc = oracle.chunked(q, k, v, g, b, cu, chunk=chunk, initial_state=s1, scale=0.5)
    assert _rel(oc, o) < 1e-12
    assert _rel(fc, f) < 1e-12


def test_literal_matrix_form_equals_scan():
    """S <- a S (I - b k k^T) + b v k^T with explicit matrices equals the rank-1 loop."""
    inp = gs.workload("tiny")
    w = inp.widened()
    args = [w[x] for x in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    rng = np.random.default_rng(12)
    s0 = rng.standard_normal((1, 2, 16, 16))
    o, f = oracle.scan(*args, initial_state=s0, scale=1.5)
    ol, fl = oracle.literal_scan(*args, initial_state=s0, scale=1.5)
    assert _rel(ol, o) < 1e-13
    assert _rel(fl, f) < 1e-13


def test_state_stays_bounded_without_decay():
    """With a = 1, b in [0, 1] and unit keys, I - b k k^T is a contraction:
    ||S_t||_F never exceeds ||S_0||_F + sum_s b_s |v_s|."""
    rng = np.random.default_rng(13)
    q, k, v, g, b, cu = _rand_inputs(rng, [200], 1, 1, 16)
    g[:] = 0.0
    s0 = rng.standard_normal((1, 1, 16, 16))
    bound = np.linalg.norm(s0)
    for t in range(0, 200, 50):
        _, f = oracle.scan(q[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], b[:t + 1],
                           np.array([0, t + 1]), initial_state=s0)
        lim = bound + np.sum(b[:t + 1, 0] * np.linalg.norm(v[:t + 1, 0], axis=-1))
        assert np.linalg.norm(f) <= lim * (1 + 1e-12)


def test_rejects_bad_arguments():
    rng = np.random.default_rng(14)
    q, k, v, g, b, cu = _rand_inputs(rng, [4], 2, 3, 8)  # hv % hk != 0
    with pytest.raises(RuntimeError):
        oracle.scan(q, k, v, g, b, cu)
    q, k, v, g, b, cu = _rand_inputs(rng, [4, 4], 1, 1, 8)
    with pytest.raises(RuntimeError):  # decreasing offsets
        oracle.scan(q, k, v, g, b, np.array([0, 9, 8]))
    with pytest.raises(ValueError):  # offsets do not end at T
        oracle.scan(q, k, v, g, b, np.array([0, 4, 7]))


# ------------------------------------------------- output normalisation pins
#
# rms_norm: y_i = o_i w_i / sqrt(mean_j o_j^2 + eps) over each row's dv values.
# A sum in place of the mean, eps outside the root, a missing root, the
# weight applied per head or reversed, or a reduction over the wrong axis
# each fails one of these.

def test_rms_norm_hand_worked():
    # o = (3, 4), w = (1, 2), eps = 0.5: mean square 12.5, + eps = 13
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.5)
    r = np.sqrt(13.0)
    assert np.allclose(y, [3.0 / r, 8.0 / r], rtol=0, atol=1e-15)


def test_rms_norm_eps_inside_the_root():
    # a constant row of ones with eps = 3 over d = 4: 1 / sqrt(1 + 3) = 1/2
    # exactly (eps outside the root, 1 / (1 + 3), would give 1/4)
    w = np.array([0.5, -1.0, 2.0, 4.0])
    y = oracle.rms_norm(np.ones(4), w, 3.0)
    assert np.array_equal(y, w / 2)


def test_rms_norm_unit_rms_per_row():
    # eps = 0, unit weights: every (token, head) row comes out with mean
    # square 1, whatever the magnitudes of the rows around it
    rng = np.random.default_rng(5)
    o = rng.standard_normal((5, 3, 8)) * (10.0 ** rng.integers(-3, 4, (5, 3, 1)))
    y = oracle.rms_norm(o, np.ones(8), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-13)
    # and each row keeps its direction
    assert np.allclose(y * np.sqrt(np.mean(o * o, axis=-1, keepdims=True)), o, rtol=1e-13, atol=0)


def test_rms_norm_one_hot_picks_its_weight():
    # a single nonzero x at channel j, eps = 0: y_j = sign(x) sqrt(d) w_j
    d = 16
    w = np.arange(1.0, d + 1.0)
    for j, x in ((0, 2.5), (7, -0.25), (15, 1e3)):
        o = np.zeros(d)
        o[j] = x
        y = oracle.rms_norm(o, w, 0.0)
        want = np.zeros(d)
        want[j] = np.sign(x) * np.sqrt(d) * w[j]
        assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_rms_norm_scale_invariant_and_zero_rows():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((4, 32))
    w = rng.standard_normal(32)
    assert np.allclose(oracle.rms_norm(-3.7 * o, w, 0.0), -oracle.rms_norm(o, w, 0.0), rtol=1e-14, atol=0)
    assert np.array_equal(oracle.rms_norm(np.zeros(32), w, 1e-6), np.zeros(32))
    assert np.isnan(oracle.rms_norm(np.zeros(32), w, 0.0)).all()
    with pytest.raises(ValueError):
        oracle.rms_norm(o, w[:31], 1e-6)


# ------------------------------------------------------ bf16 rounding pins
#
# round_to_bf16 rounds float64 to the nearest bfloat16 (8 significant bits),
# ties to even. Hand-worked values fix the tie rule and the scale; the
# storage generator's independent float32 -> bf16 bit routine fixes every
# exponent range it covers.

def test_round_to_bf16_hand_worked():
    r = oracle.round_to_bf16
    # spacing at 1 is 2^-7: 1 + 2^-8 is a tie (to the even 1.0); 1 + 3 2^-8
    # lies between 1 + 2^-7 (odd) and 1 + 2^-6 (even) on a tie too
    assert r(1 + 2.0 ** -8) == 1.0
    assert r(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert r(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    assert r(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7  # just past the tie
    assert r(0.1) == 0.10009765625  # 0x3DCD
    assert r(2.0 ** -130) == 2.0 ** -130  # subnormal, exact
    big = (2 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16
    assert r(big) == big
    assert r(big + 2.0 ** 119 - 2.0 ** 100) == big  # below the tie with 2^128
    assert r(big + 2.0 ** 119) == np.inf  # the tie rounds to even: 2^128 overflows
    assert r(0.0) == 0.0 and np.isnan(r(np.nan))


def test_round_to_bf16_matches_bit_rounding_of_float32():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    want = gs.bf16_bits_to_f32(gs.f32_to_bf16_bits(x)).astype(np.float64)
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # idempotent and monotone
    assert np.array_equal(oracle.round_to_bf16(got), got)
    xs = np.sort(x.astype(np.float64))
    assert np.all(np.diff(oracle.round_to_bf16(xs)) >= 0)
