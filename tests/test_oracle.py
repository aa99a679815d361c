"""Pins of the CPU oracle against things other than itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a wrong head map, > instead of >=)
fails at least one test: exact rational brute force for pooling, the dense
logit-tile mean for the block score, the threshold's closed-form special
cases (gamma = 0 and gamma = 1), nesting in gamma, the geometric-mean reading
of the cross-query average, dense causal softmax attention for gamma = 0,
brute-force masked attention on tiny inputs, and the hand-worked example in
tests/golden.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import gen
import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def small_case(dtype="bf16", hq=4, hkv=2, seq=256, d=16, block=32, seed=0, **kw):
    return gen.make_case(hq, hkv, seq, d, block, dtype, seed, **kw)


# ---------------------------------------------------------------- decoding
def test_decode_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3fn(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_e4m3fn_format_points():
    # values fixed by the OCP e4m3fn definition
    assert oracle.decode_e4m3fn(0x7E) == 448.0
    assert oracle.decode_e4m3fn(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3fn(0x01) == 2.0 ** -9
    assert oracle.decode_e4m3fn(0x07) == 7 * 2.0 ** -9
    assert oracle.decode_e4m3fn(0x38) == 1.0
    assert oracle.decode_e4m3fn(0xB8) == -1.0
    assert oracle.decode_e4m3fn(0x3C) == 1.5


def test_decode_bf16_matches_torch():
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


# ---------------------------------------------------------------- pooling
def test_pool_exact_rational_bf16():
    c = small_case("bf16", hq=2, hkv=1, seq=96, d=4, block=32, seed=3, n_vert=3)
    got = oracle.pool(c.q, "bf16", c.block)
    vals = brute.decode(c.q, "bf16")
    for h in range(2):
        for I in range(3):
            for e in range(4):
                s = sum(Fraction(float(vals[h, t, e])) for t in range(I * 32, I * 32 + 32))
                assert Fraction(got[h, I, e]) == s / 32


def test_pool_ragged_tail_means_valid_tokens():
    x = np.arange(2 * 70 * 3, dtype=np.float32).reshape(2, 70, 3) * 0.25
    got = oracle.pool(x, "f32", 32)
    assert got.shape == (2, 3, 3)
    np.testing.assert_allclose(got[:, 2], x[:, 64:70].astype(np.float64).mean(1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[:, 0], x[:, :32].astype(np.float64).mean(1), rtol=0, atol=1e-12)


def test_pool_fp8_is_mean_of_dequantised():
    c = small_case("fp8", hq=2, hkv=1, seq=128, d=8, block=64, seed=5, n_vert=2)
    q = brute.decode(c.q, "fp8", c.q_scale)
    got = oracle.pool(c.q, "fp8", 64, c.q_scale)
    np.testing.assert_allclose(got, q.reshape(2, 2, 64, 8).mean(2), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- score
@pytest.mark.parametrize("dtype,hq,hkv", [("f32", 2, 1), ("bf16", 4, 2), ("bf16", 4, 4), ("fp8", 6, 2)])
def test_score_equals_mean_of_dense_logit_tile(dtype, hq, hkv):
    c = small_case(dtype, hq=hq, hkv=hkv, seq=192, d=16, block=32, seed=11, n_vert=4)
    q, k, _ = brute.values(c)
    cs = brute.sm(c.d)
    tile = brute.block_tile_mean_logits(q, k, hq, hkv, cs, c.block)
    qb = oracle.pool(c.q, dtype, c.block, c.q_scale)
    kb = oracle.pool(c.k, dtype, c.block, c.k_scale)
    S, P = oracle.score(qb, kb, cs)
    nb = c.nb
    low = np.tril(np.ones((nb, nb), bool))
    np.testing.assert_allclose(S[:, low], tile[:, low], rtol=1e-10, atol=1e-12)
    assert np.all(S[:, ~low] == 0) and np.all(P[:, ~low] == 0)
    np.testing.assert_allclose(P, brute.causal_softmax_rows(np.where(low, tile, 0)), rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)


def test_score_head_map_is_contiguous_groups():
    # kv head 1 gets a huge planted key block; only q heads 2,3 (group 1) may see it
    c = small_case("f32", hq=4, hkv=2, seq=128, d=8, block=32, seed=2)
    c.k[1, 32:64] += 10.0
    c.q[:] += 1.0
    qb = oracle.pool(c.q, "f32", 32)
    kb = oracle.pool(c.k, "f32", 32)
    S, _ = oracle.score(qb, kb, 1.0)
    tile = brute.block_tile_mean_logits(brute.decode(c.q, "f32"), brute.decode(c.k, "f32"), 4, 2, 1.0, 32)
    low = np.tril(np.ones((4, 4), bool))
    np.testing.assert_allclose(S[:, low], tile[:, low], atol=1e-10)
    assert S[2, 3, 1] > S[0, 3, 1] + 10


# ---------------------------------------------------------------- mask
def _pipeline(c, gamma, sink=1, local=1):
    cs = brute.sm(c.d)
    qb = oracle.pool(c.q, c.dtype, c.block, c.q_scale)
    kb = oracle.pool(c.k, c.dtype, c.block, c.k_scale)
    S, P = oracle.score(qb, kb, cs)
    return S, P, oracle.mask(P, gamma, sink, local)


def test_mask_gamma0_is_full_causal():
    c = gen.make_s1(0)
    _, P, (m, idx, cnt) = _pipeline(c, 0.0)
    nb = c.nb
    assert np.array_equal(m, np.broadcast_to(np.tril(np.ones((nb, nb), np.uint8)), m.shape))
    assert np.array_equal(cnt, np.broadcast_to(np.arange(1, nb + 1), cnt.shape))


def test_mask_gamma1_is_argmax_sink_diag():
    c = gen.make_s1(1)
    S, P, (m, idx, cnt) = _pipeline(c, 1.0, sink=1, local=1)
    nb = c.nb
    for h in range(c.hq):
        for I in range(nb):
            row = S[h, I, :I + 1]
            want = set(np.flatnonzero(row == row.max()).tolist()) | {0, I}
            assert set(np.flatnonzero(m[h, I]).tolist()) == want


def test_mask_threshold_against_log_form_and_band():
    # P >= gamma * Pmax  <=>  S - max S >= ln gamma   (outside a tiny band)
    for seed in range(4):
        c = gen.make_s1(seed)
        S, P, (m, idx, cnt) = _pipeline(c, c.gamma, sink=0, local=0)
        nb = c.nb
        for I in range(nb):
            s = S[:, I, :I + 1]
            d = s - s.max(-1, keepdims=True) - math.log(c.gamma)
            sure = np.abs(d) > 1e-9
            assert np.array_equal((d >= 0)[sure], m[:, I, :I + 1].astype(bool)[sure])
        dens = m.sum() / (c.hq * nb * (nb + 1) / 2)
        assert 0.05 < dens < 0.95, dens  # S1 masks are nonuniform


def test_mask_ties_are_kept_and_compaction():
    P = np.zeros((1, 4, 4))
    P[0, 0, 0] = 1
    P[0, 1, :2] = [0.5, 0.5]
    P[0, 2, :3] = [0.4, 0.2, 0.4]
    P[0, 3, :4] = [0.1, 0.45, 0.0, 0.45]
    m, idx, cnt = oracle.mask(P, 0.5, 0, 0)
    assert m[0].tolist() == [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [0, 1, 0, 1]]
    assert cnt[0].tolist() == [1, 2, 3, 2]
    assert idx[0, 3].tolist() == [1, 3, -1, -1]
    m, idx, cnt = oracle.mask(P, 1.0, 0, 0)
    assert m[0, 3].tolist() == [0, 1, 0, 1] and m[0, 2].tolist() == [1, 0, 1, 0]
    # sink and local windows are ORed in; local counts blocks ending at the diagonal
    m, idx, cnt = oracle.mask(P, 1.0, 1, 2)
    assert m[0, 3].tolist() == [1, 1, 1, 1] and m[0, 2].tolist() == [1, 1, 1, 0]


def test_mask_nesting_in_gamma_and_forced_blocks():
    c = gen.make_s1(2)
    prev = None
    for g in [0.0, 0.01, 0.05, 0.1, 0.3, 0.6, 1.0]:
        _, P, (m, idx, cnt) = _pipeline(c, g)
        nb = c.nb
        assert np.all(m[:, :, 0] == 1)
        assert np.all(m[:, np.arange(nb), np.arange(nb)] == 1)
        # row argmax always kept
        am = np.argmax(np.where(np.tril(np.ones((nb, nb), bool)), P, -1), axis=-1)
        assert np.all(np.take_along_axis(m, am[..., None], -1) == 1)
        if prev is not None:
            assert np.all(m <= prev)  # larger gamma keeps a subset
        prev = m
        for h in range(c.hq):
            for I in range(nb):
                assert idx[h, I, :cnt[h, I]].tolist() == np.flatnonzero(m[h, I]).tolist()


# ---------------------------------------------------------------- arithmetic scorer
def test_score_arith_block1_is_causal_attention_probabilities():
    """With one token per block, the block average is the token itself and
    pooled keys are the keys: the scorer is textbook causal softmax."""
    rng = np.random.default_rng(5)
    hq, hkv, seq, d = 4, 2, 40, 8
    q = rng.standard_normal((hq, seq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, seq, d)).astype(np.float32)
    c = 0.37
    P = oracle.score_arith(q, k, "f32", 1, c, hkv)
    L = brute.dense_logits(q.astype(np.float64), k.astype(np.float64), hq, hkv, c)
    L = np.where(np.tril(np.ones((seq, seq), bool))[None], L, -np.inf)
    e = np.exp(L - L.max(-1, keepdims=True))
    np.testing.assert_allclose(P, e / e.sum(-1, keepdims=True), rtol=1e-12, atol=1e-15)


def test_score_arith_rows_sum_to_one_with_ragged_tail():
    c = small_case("bf16", seq=250, block=32, seed=3)
    P = oracle.score_arith(c.q, c.k, c.dtype, c.block, brute.sm(c.d), c.hkv)
    nb = P.shape[1]
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(P[:, np.triu_indices(nb, 1)[0], np.triu_indices(nb, 1)[1]] == 0)
    assert np.all(P >= 0)


def test_score_arith_bounds_the_geometric_mean_and_meets_it_for_equal_queries():
    """The block score is the arithmetic mean of the queries' probabilities;
    their geometric mean is exp(c Qbar.Kbar_J - mean_i LSE_i) (the pooled-query
    reading), so the scorer is never below it, and equal for equal queries."""
    c = small_case("f32", hq=2, hkv=1, seq=256, d=16, block=32, seed=4)
    cs = brute.sm(c.d)
    q = brute.decode(c.q, "f32")
    kb = oracle.pool(c.k, "f32", c.block)
    P = oracle.score_arith(c.q, c.k, "f32", c.block, cs, c.hkv)
    nb = kb.shape[1]
    for h in range(2):
        for I in range(nb):
            qi = q[h, I * c.block:(I + 1) * c.block]
            s = cs * qi @ kb[0, :I + 1].T
            lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
            gm = np.exp((s - lse[:, None]).mean(0))
            assert np.all(gm <= P[h, I, :I + 1] * (1 + 1e-12))
    # every query of a block equal to the block mean: arithmetic = pooled score
    qe = c.q.copy()
    for I in range(nb):
        qe[:, I * c.block:(I + 1) * c.block] = qe[:, I * c.block:(I + 1) * c.block].mean(1,
                                                                                         keepdims=True)
    Pe = oracle.score_arith(qe, c.k, "f32", c.block, cs, c.hkv)
    _, Pp = oracle.score(oracle.pool(qe, "f32", c.block), kb, cs)
    np.testing.assert_allclose(Pe, Pp, rtol=1e-9, atol=1e-13)


def test_score_arith_fp8_equals_f32_on_dequantised_and_rows_subset():
    c = small_case("fp8", seq=256, block=64, seed=6)
    cs = brute.sm(c.d)
    P8 = oracle.score_arith(c.q, c.k, "fp8", c.block, cs, c.hkv, c.q_scale, c.k_scale)
    qf = brute.decode(c.q, "fp8", c.q_scale).astype(np.float32)
    kf = brute.decode(c.k, "fp8", c.k_scale).astype(np.float32)
    Pf = oracle.score_arith(qf, kf, "f32", c.block, cs, c.hkv)
    np.testing.assert_allclose(P8, Pf, rtol=1e-6, atol=1e-9)  # f32 rounding of code * scale
    rows = np.array([0, 3, 5, 9], np.int64)
    nb = P8.shape[1]
    np.testing.assert_array_equal(
        oracle.score_arith(c.q, c.k, "fp8", c.block, cs, c.hkv, c.q_scale, c.k_scale, rows=rows),
        P8.reshape(-1, nb)[rows])


# ---------------------------------------------------------------- rescue branch
def test_key_radius_closed_forms():
    rng = np.random.default_rng(11)
    hkv, block, d = 2, 16, 8
    seq = 5 * block + 6  # ragged tail of 6 keys
    k = np.empty((hkv, seq, d), np.float32)
    a = rng.standard_normal((hkv, 6, d)).astype(np.float32)
    b = rng.standard_normal((hkv, 6, d)).astype(np.float32)
    for J in range(6):
        t0, t1 = J * block, min((J + 1) * block, seq)
        n = t1 - t0
        k[:, t0:t1] = a[:, J:J + 1]
        if J % 2:  # two-point block: half the keys at a, half at b
            k[:, t0 + n // 2:t1] = b[:, J:J + 1]
    r = oracle.key_radius(k, "f32", block)
    for J in range(6):
        want = 0.0 if J % 2 == 0 else np.linalg.norm(a[:, J].astype(np.float64) - b[:, J], axis=-1) / 2
        np.testing.assert_allclose(r[:, J], want, rtol=1e-6, atol=1e-6)
    # translating every key of a block leaves its radius unchanged
    x = rng.standard_normal((hkv, 4 * block, d)).astype(np.float32)
    r1 = oracle.key_radius(x, "f32", block)
    r2 = oracle.key_radius(x + np.float32(3.0), "f32", block)
    np.testing.assert_allclose(r1, r2, rtol=1e-5)


def test_rescue_score_bounds_every_key_and_is_tight_along_the_query():
    c = small_case("f32", hq=2, hkv=1, seq=128, d=8, block=16, seed=12)
    cs = brute.sm(c.d)
    qb = oracle.pool(c.q, "f32", c.block)
    kb = oracle.pool(c.k, "f32", c.block)
    r = oracle.key_radius(c.k, "f32", c.block)
    R, Pr = oracle.score_rescue(qb, kb, r, cs)
    k = brute.decode(c.k, "f32")
    nb = qb.shape[1]
    for h in range(2):
        for I in range(nb):
            for J in range(I + 1):
                best = (cs * k[0, J * c.block:(J + 1) * c.block] @ qb[h, I]).max()
                assert R[h, I, J] >= best - 1e-9
    np.testing.assert_allclose(Pr.sum(-1), 1.0, atol=1e-12)
    # keys of block 2 at its mean +- t * u, u along Qbar of row (0, 5): the bound is reached
    k2 = c.k.copy()
    u = qb[0, 5] / np.linalg.norm(qb[0, 5])
    mvec = kb[0, 2]
    t = 0.75
    k2[0, 2 * c.block:3 * c.block:2] = (mvec + t * u).astype(np.float32)
    k2[0, 2 * c.block + 1:3 * c.block:2] = (mvec - t * u).astype(np.float32)
    kb2 = oracle.pool(k2, "f32", c.block)
    r2 = oracle.key_radius(k2, "f32", c.block)
    R2, _ = oracle.score_rescue(qb, kb2, r2, cs)
    best = (cs * brute.decode(k2, "f32")[0, 2 * c.block:3 * c.block] @ qb[0, 5]).max()
    np.testing.assert_allclose(R2[0, 5, 2], best, rtol=1e-6)


def test_mask_dual_union_and_zero_radius_reduction():
    c = gen.make_s1(2)
    cs = brute.sm(c.d)
    qb = oracle.pool(c.q, c.dtype, c.block)
    kb = oracle.pool(c.k, c.dtype, c.block)
    _, P = oracle.score(qb, kb, cs)
    r = oracle.key_radius(c.k, c.dtype, c.block)
    _, Pr = oracle.score_rescue(qb, kb, r, cs)
    for g, gr in [(0.1, 0.3), (0.3, 0.05), (1.0, 1.0)]:
        m, idx, cnt = oracle.mask_dual(P, Pr, g, gr)
        mb = oracle.mask(P, g)[0]
        mr = oracle.mask(Pr, gr)[0]
        assert np.array_equal(m, mb | mr)
        for h in range(c.hq):
            for I in range(c.nb):
                assert idx[h, I, :cnt[h, I]].tolist() == np.flatnonzero(m[h, I]).tolist()
    # no radius: the rescue branch is the base score, the union is the laxer threshold
    _, P0 = oracle.score_rescue(qb, kb, np.zeros_like(r), cs)
    np.testing.assert_allclose(P0, P, rtol=1e-12, atol=1e-15)
    for g, gr in [(0.1, 0.4), (0.5, 0.2)]:
        assert np.array_equal(oracle.mask_dual(P, P0, g, gr)[0], oracle.mask(P, min(g, gr))[0])


def _exhaustive_calibration(P, target, sink, local):
    """Exhaustive answer: density only changes at the ratios P / row max, so
    try every candidate (each distinct ratio of a causal block, and 1),
    count the kept blocks at it, and keep the largest candidate whose kept
    share reaches the target.  No sorting or order statistic."""
    hq, nb, _ = P.shape
    I = np.arange(nb)[:, None]
    J = np.arange(nb)[None, :]
    causal = J <= I
    forced = causal & ((J < sink) | (I - J < local))
    pmax = np.where(causal, P, -np.inf).max(-1, keepdims=True)
    ratios = np.where(causal, P / pmax, np.nan)
    total = hq * nb * (nb + 1) / 2

    def dens(g):
        return ((causal & (ratios >= g)) | forced).sum() / total

    if dens(1.0) >= target:
        return 1.0
    best = 0.0
    for r in np.unique(ratios[~np.isnan(ratios)]):
        if r <= 1.0 and dens(r) >= target:
            best = max(best, r)
    return best


@pytest.mark.parametrize("seed,target,sink,local", [(0, 0.3, 1, 1), (1, 0.5, 1, 1),
                                                     (2, 0.7, 1, 1), (3, 0.9, 1, 1),
                                                     (0, 0.05, 1, 1), (1, 0.6, 2, 4),
                                                     (2, 0.4, 4, 8), (3, 0.8, 0, 0)])
def test_calibrate_gamma_is_the_exact_answer(seed, target, sink, local):
    c = gen.make_s1(seed)
    _, P, _ = _pipeline(c, 0.1)
    g, d = oracle.calibrate_gamma(P, target, sink, local)
    exact = _exhaustive_calibration(P, target, sink, local)
    assert g == exact
    total = c.hq * c.nb * (c.nb + 1) / 2
    # the oracle's own mask reaches the target at gamma and misses it just above
    _, _, cnt = oracle.mask(P, g * (1 - 1e-12), sink, local)
    assert cnt.sum() / total >= target and abs(cnt.sum() / total - d) < 1e-12
    if g < 1.0:
        _, _, cnt = oracle.mask(P, g * (1 + 1e-9), sink, local)
        assert cnt.sum() / total < target


def test_calibrate_gamma_edges_and_monotone_in_target():
    c = gen.make_s1(1)
    _, P, _ = _pipeline(c, 0.1)
    assert oracle.calibrate_gamma(P, 1.0)[1] == 1.0
    # forced blocks alone reach a tiny target: gamma 1
    assert oracle.calibrate_gamma(P, 1e-3) == (1.0, oracle.calibrate_gamma(P, 1e-3)[1])
    gs = [oracle.calibrate_gamma(P, t)[0] for t in (0.2, 0.4, 0.6, 0.8, 0.95)]
    assert all(a >= b for a, b in zip(gs, gs[1:]))
    # wider structural retention never needs a smaller gamma for the same target
    assert oracle.calibrate_gamma(P, 0.6, sink_blocks=3, local_blocks=3)[0] >= gs[2]


def test_user_mask_is_anded_with_causal_without_forced_blocks():
    rng = np.random.default_rng(0)
    um = (rng.random((3, 8, 8)) < 0.4).astype(np.uint8)
    m, idx, cnt = oracle.mask(None, 0.5, 1, 1, user_mask=um)
    assert np.array_equal(m, um & np.tril(np.ones((8, 8), np.uint8)))
    assert np.array_equal(cnt, m.sum(-1))


def test_pooled_query_mask_equals_geometric_mean_reading():
    """Section 3 of the page calls exp(q . Kbar) a geometric-mean proxy and
    averages across the queries of a block.  Reading that average as a
    geometric mean of per-query softmax probabilities gives
    exp(c Qbar_I . Kbar_J - mean_i LSE_i), whose row-max threshold equals the
    pooled-Q threshold exactly."""
    for seed in range(3):
        c = gen.make_s1(seed)
        q, k, _ = brute.values(c)
        cs = brute.sm(c.d)
        kb = oracle.pool(c.k, c.dtype, c.block)
        _, _, (m, _, _) = _pipeline(c, c.gamma, sink=0, local=0)
        nb, B = c.nb, c.block
        for h in range(c.hq):
            for I in range(nb):
                lg = cs * q[h, I * B:(I + 1) * B] @ kb[0, :I + 1].T  # [B, I+1]
                lse = np.log(np.exp(lg - lg.max(1, keepdims=True)).sum(1)) + lg.max(1)
                logp = lg - lse[:, None]
                geo = logp.mean(0)  # log of the geometric mean over i in I
                d = geo - geo.max() - math.log(c.gamma)
                sure = np.abs(d) > 1e-9
                assert np.array_equal((d >= 0)[sure], m[h, I, :I + 1].astype(bool)[sure])


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_attn_gamma0_is_dense_causal_softmax(dtype):
    c = small_case(dtype, hq=4, hkv=2, seq=160, d=16, block=32, seed=7, n_vert=3)
    res = oracle.prefill(c, gamma=0.0)
    assert res["mask"].sum() == c.hq * c.nb * (c.nb + 1) // 2
    q, k, v = brute.values(c)
    causal = np.broadcast_to(np.tril(np.ones((c.seq, c.seq), bool)), (c.hq, c.seq, c.seq))
    out, lse = brute.attention(q, k, v, c.hq, c.hkv, brute.sm(c.d), causal)
    np.testing.assert_allclose(res["out"], out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attn_brute_force_random_masks(seed):
    c = small_case("bf16", hq=4, hkv=1, seq=200, d=8, block=32, seed=seed)  # ragged tail
    nb = c.nb
    rng = np.random.default_rng(seed)
    bm = (rng.random((c.hq, nb, nb)) < 0.5).astype(np.uint8)
    bm[0, 3, :] = 0  # one empty row
    q, k, v = brute.values(c)
    out, lse = oracle.attn(c.q, c.k, c.v, "bf16", c.block, bm)
    rout, rlse = brute.attention(q, k, v, c.hq, c.hkv, brute.sm(c.d), brute.token_mask(bm, c.seq, c.block))
    np.testing.assert_allclose(out, rout, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(rlse))
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(lse[fin], rlse[fin], rtol=1e-12, atol=1e-12)
    assert np.all(out[0, 96:128] == 0) and np.all(np.isneginf(lse[0, 96:128]))


def test_attn_rows_sum_to_one_and_sampled_rows():
    c = small_case("f32", hq=2, hkv=1, seq=128, d=8, block=32, seed=4)
    c.v[:] = 1.0
    bm = np.tril(np.ones((2, 4, 4), np.uint8))
    bm[:, 3, 1] = 0
    out, lse = oracle.attn(c.q, c.k, c.v, "f32", 32, bm)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    rows = np.array([5, 127, 128 + 100, 255], np.int64)
    o2, l2 = oracle.attn(c.q, c.k, c.v, "f32", 32, bm, rows=rows)
    np.testing.assert_array_equal(o2, out.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(l2, lse.reshape(-1)[rows])


def test_attn_diagonal_only_is_blockwise_local_causal():
    c = small_case("bf16", hq=2, hkv=2, seq=128, d=8, block=32, seed=9)
    q, k, v = brute.values(c)
    bm = np.broadcast_to(np.eye(4, dtype=np.uint8), (2, 4, 4)).copy()
    out, _ = oracle.attn(c.q, c.k, c.v, "bf16", 32, bm)
    for h in range(2):
        for I in range(4):
            sl = slice(I * 32, I * 32 + 32)
            lg = brute.sm(8) * q[h, sl] @ k[h, sl].T
            lg = np.where(np.tril(np.ones((32, 32), bool)), lg, -np.inf)
            p = np.exp(lg - lg.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            np.testing.assert_allclose(out[h, sl], p @ v[h, sl], rtol=1e-12, atol=1e-13)


def test_attn_duplicated_q_heads_and_mha():
    c = small_case("bf16", hq=4, hkv=2, seq=96, d=8, block=32, seed=12)
    c.q[1] = c.q[0]
    c.q[3] = c.q[2]
    bm = np.tril(np.ones((4, 3, 3), np.uint8))
    out, lse = oracle.attn(c.q, c.k, c.v, "bf16", 32, bm)
    np.testing.assert_array_equal(out[0], out[1])
    np.testing.assert_array_equal(out[2], out[3])
    # MHA view of the same problem: expand kv heads to hq
    k4 = np.repeat(c.k, 2, axis=0)
    v4 = np.repeat(c.v, 2, axis=0)
    out4, _ = oracle.attn(c.q, k4, v4, "bf16", 32, bm)
    np.testing.assert_array_equal(out, out4)


def test_attn_fp8_equals_f32_on_dequantised():
    c = small_case("fp8", hq=4, hkv=2, seq=128, d=16, block=32, seed=13, n_vert=2)
    q, k, v = brute.values(c)
    bm = np.tril(np.ones((4, 4, 4), np.uint8))
    o8, l8 = oracle.attn(c.q, c.k, c.v, "fp8", 32, bm, q_scale=c.q_scale, k_scale=c.k_scale,
                         v_scale=c.v_scale)
    # the f32 path sees the dequantised values rounded once to float32, so the two
    # agree to float32 rounding of the inputs
    of, lf = oracle.attn(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), "f32",
                         32, bm)
    np.testing.assert_allclose(o8, of, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(l8, lf, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- worked example
def _ev(x):
    return np.vectorize(lambda s: float(eval(s, {"math": math, "__builtins__": {}})))(np.array(x, dtype=object))


def test_worked_example_from_golden():
    g = json.load(open(GOLDEN))
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    v = np.array(g["v"], np.float32)
    B = g["shape"]["block"]
    qb = oracle.pool(q, "f32", B)
    kb = oracle.pool(k, "f32", B)
    np.testing.assert_allclose(qb, _ev(g["qbar"]), atol=1e-15)
    np.testing.assert_allclose(kb, _ev(g["kbar"]), atol=1e-15)
    S, P = oracle.score(qb, kb, g["shape"]["sm_scale"])
    np.testing.assert_allclose(S, _ev(g["S"]), atol=1e-15)
    np.testing.assert_allclose(P, _ev(g["P"]), rtol=1e-14, atol=1e-15)
    for cs in g["cases"]:
        m, idx, cnt = oracle.mask(P, cs["gamma"], cs["sink_blocks"], cs["local_blocks"])
        assert m.tolist() == cs["mask"]
        out, lse = oracle.attn(q, k, v, "f32", B, m, g["shape"]["sm_scale"])
        np.testing.assert_allclose(out, _ev(cs["out"]), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse, _ev(cs["lse"]), rtol=1e-14, atol=1e-15)
