"""Pins of the price router's oracle (Triage: per-tier error predicted from
block statistics, one price).  The error model is this implementation's
reading of a one-sentence description, so as a predictor it is parity
unpinned; what is pinned here is everything that has an independent
definition: the block statistics (brute-force loops, numpy's variance), the
score-spread identity on keys whose deviations are uncorrelated across
dimensions, the model's zero where the skip tier is exact, the skip error
against a direct simulation of the quantities it predicts, the fp8 score
noise against real E4M3 rounding, and the structure of the decision rule."""
import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import FULL, LOW, SKIP
from oracle import tattn as T


def cfg(bq, bk, price, mode=4):
    return SimpleNamespace(block_q=bq, block_k=bk, tau_hi=0.05, tau_lo=0.005, top_k=0, mode=mode,
                           keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256, price=price)


def test_block_moments_brute_force():
    """Per-block mean square, variance, their totals and the mean's norm,
    from scalar loops over a ragged blocking."""
    r = np.random.default_rng(1)
    n, d, b = 37, 5, 16
    x = (r.standard_normal((n, d)) * 1.7 + 0.4).astype(np.float32)
    m = T.block_moments(x, b)
    for j in range(3):
        rows = range(j * b, min(n, (j + 1) * b))
        sz = len(rows)
        tm2 = tv = mn = 0.0
        for c in range(d):
            s1 = s2 = 0.0
            for i in rows:
                s1 += float(x[i, c])
                s2 += float(x[i, c]) ** 2
            msq, mean = s2 / sz, s1 / sz
            var = max(msq - mean * mean, 0.0)
            assert m["m2"][j, c] == pytest.approx(msq, rel=2 ** -23)
            assert m["var"][j, c] == pytest.approx(var, rel=2 ** -22)
            assert m["var"][j, c] == pytest.approx(np.var(x[list(rows), c].astype(np.float64)), rel=2 ** -22)
            tm2 += msq
            tv += var
            mn += mean * mean
        assert m["tot_m2"][j] == pytest.approx(tm2, rel=2 ** -23)
        assert m["tot_var"][j] == pytest.approx(tv, rel=2 ** -22)
        assert m["mnorm"][j] == pytest.approx(math.sqrt(mn), rel=2 ** -23)


def test_score_spread_identity_for_axis_deviations():
    """Keys k_J +- a_c e_c (pairs along distinct axes) have uncorrelated
    deviations, so the mean square of q_i.(k_j - k_J)/sqrt(d) over the tile's
    pairs equals sum_c q2_c var_c / d exactly."""
    r = np.random.default_rng(2)
    d, bq, bk = 8, 8, 16
    q = r.standard_normal((bq, d)).astype(np.float32)
    center = r.standard_normal(d)
    k = np.empty((bk, d), np.float32)
    for j in range(bk):
        c = (j // 2) % d
        k[j] = center
        k[j, c] += (1.0 if j % 2 == 0 else -1.0) * (0.25 + 0.125 * c)
    qm, km = T.block_moments(q, bq), T.block_moments(k, bk)
    s2 = T.tile_error_model(qm["m2"], qm["tot_m2"], km["var"], km["tot_m2"], km["tot_var"], km["tot_m2"],
                            km["mnorm"], np.array([bk]), d)[0]
    kd = k.astype(np.float64) - k.astype(np.float64).mean(axis=0)
    delta = (q.astype(np.float64) @ kd.T) / math.sqrt(d)
    assert s2[0, 0] == pytest.approx(float((delta ** 2).mean()), rel=1e-6)


@pytest.mark.parametrize("price", [0.0, 1e-6, 1e-2, 10.0])
def test_skip_error_vanishes_where_skip_is_exact(price):
    """Keys constant inside every key block: the skip tier is exact (pin P2),
    and the model predicts zero skip error, so every off-diagonal tile is
    skipped at any price and the output equals textbook attention."""
    r = np.random.default_rng(3)
    n, d, bq, bk = 200, 16, 64, 32
    q = r.standard_normal((n, d)).astype(np.float32)
    kc = r.standard_normal((-(-n // bk), d)).astype(np.float32)
    k = np.repeat(kc, bk, axis=0)[:n]
    v = r.standard_normal((n, d)).astype(np.float32)
    c = cfg(bq, bk, price)
    plan = T.oracle_plan(q, k, v, c)
    assert np.all(plan["price"]["eS"] == 0.0)
    diag = T.diagonal_mask(n, bq, bk)
    assert np.all(plan["tiers"][~diag] == SKIP)
    out = T.oracle_forward(q, k, v, plan, bq, bk)
    assert np.abs(out - T.naive_attention(q, k, v)).max() < 1e-6   # block means are stored in float32


def test_skip_error_against_direct_simulation():
    """Draw one tile many times (Gaussian key deviations, independent values),
    compute what skipping it changes -- the mass ratio n_J / sum w and the
    distance of the weighted value mean from the block mean -- and compare
    with the model's two skip terms fed with each draw's own statistics."""
    r = np.random.default_rng(4)
    d, n, trials = 16, 64, 3000
    q = (r.standard_normal(d) * 1.3).astype(np.float32)[None, :]
    ksd = np.linspace(0.2, 0.9, d)
    mass, dist2, mass_m, dist2_m = [], [], [], []
    for _ in range(trials):
        k = (r.standard_normal((n, d)) * ksd).astype(np.float32)
        v = r.standard_normal((n, d)).astype(np.float32)
        w = np.exp((q.astype(np.float64) @ (k - k.astype(np.float64).mean(axis=0)).T)[0] / math.sqrt(d))
        o = (w[:, None] * v.astype(np.float64)).sum(axis=0) / w.sum()
        mass.append(n / w.sum())
        dist2.append(float(((o - v.astype(np.float64).mean(axis=0)) ** 2).sum()))
        qm, km, vm = T.block_moments(q, 1), T.block_moments(k, n), T.block_moments(v, n)
        s2 = float((qm["m2"][0].astype(np.float64) * km["var"][0]).sum() / d)
        mass_m.append(math.exp(-0.5 * s2))
        dist2_m.append(float(vm["tot_var"][0]) * math.expm1(s2) / n)
    assert np.mean(mass) == pytest.approx(np.mean(mass_m), rel=0.03)
    assert np.mean(dist2) == pytest.approx(np.mean(dist2_m), rel=0.10)


def test_low_score_noise_bounds_real_e4m3_rounding():
    """The fp8 score-noise variance (2u^2/3) m2q m2k / d^2 assumes every
    element is off by up to half an E4M3 ulp; real rounding of Gaussian data
    (through the oracle's own quantiser) must come out below it, and within a
    factor of 3."""
    r = np.random.default_rng(5)
    d, b = 64, 64
    q = r.standard_normal((b, d)).astype(np.float32)
    k = (r.standard_normal((b, d)) * 0.7 + 0.2).astype(np.float32)
    q8, sq, _ = T.quantise_blocks(q, b)
    k8, sk, _ = T.quantise_blocks(k, b)
    from oracle import e4m3
    qh = e4m3.decode(q8) * float(sq[0])
    kh = e4m3.decode(k8) * float(sk[0])
    err = (qh @ kh.T - q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
    qm, km = T.block_moments(q, b), T.block_moments(k, b)
    sl2 = (2.0 * T.E4M3_U ** 2 / 3.0) * float(qm["tot_m2"][0]) * float(km["tot_m2"][0]) / d ** 2
    ratio = float((err ** 2).mean()) / sl2
    assert 1.0 / 3.0 <= ratio <= 1.0, ratio


def _rank(t):
    return np.asarray(t, np.int64)   # SKIP 0 < LOW 1 < FULL 2: cost order


def test_price_rule_structure():
    """Raising the price never moves a tile to a more accurate tier; at price
    0 every tile with a predicted error is FULL; at a prohibitive price every
    tile is skipped; every tile takes the minimum of its three objectives."""
    r = np.random.default_rng(6)
    n, d, bq, bk = 512, 32, 64, 32
    q, k, v = [r.standard_normal((n, d)).astype(np.float32) for _ in range(3)]
    base = T.oracle_plan(q, k, v, cfg(bq, bk, 0.0))
    info, p = base["price"], base["price"]["pt"]
    prev = None
    for lam in [0.0, 1e-5, 1e-4, 1e-3, 1e-2, 1e-1, 1.0, 1e3]:
        t, (oS, oL, oF) = T.tiers_price(p, info["eS"], info["eL"], lam, bk)
        objs = np.stack([oS, oL, oF])
        assert np.all(np.take_along_axis(objs, _rank(t)[None], 0)[0] == objs.min(axis=0))
        if prev is not None:
            assert np.all(_rank(t) <= _rank(prev))
        prev = t
        if lam == 0.0:
            assert np.all(t[(p * info["eS"] > 0) & (p * info["eL"] > 0)] == FULL)
        if lam == 1e3:
            assert np.all(t == SKIP)
    # the tie rule: equal objectives go to the cheaper tier
    t, _ = T.tiers_price(np.zeros((1, 3)), np.zeros((1, 3)), np.zeros((1, 3)), 0.0, bk)
    assert np.all(t == SKIP)


def test_price_plan_forces_the_diagonal_and_partitions_lists():
    r = np.random.default_rng(7)
    n, d, bq, bk = 300, 16, 128, 64
    q, k, v = [r.standard_normal((n, d)).astype(np.float32) for _ in range(3)]
    plan = T.oracle_plan(q, k, v, cfg(bq, bk, 1e3))
    diag = T.diagonal_mask(n, bq, bk)
    assert np.all(plan["tiers"][diag] == FULL) and np.all(plan["tiers"][~diag] == SKIP)
    assert np.all(plan["counts"].sum(axis=1) == plan["tiers"].shape[1])


def test_skim_score_noise_bounds_real_mxfp4_rounding():
    """The SKIM tier's score-noise variance (2u^2/3) m2q m2k / d^2 with
    u = 2^-2: real MXFP4 rounding of Gaussian data (through the oracle's own
    codec, one scale per 32 channels) must come out below it, and within a
    factor of 3; so must the value error against u sqrt(m2v/3)."""
    from oracle import mxfp4
    for seed in range(3):
        r = np.random.default_rng(50 + seed)
        d, b = 64, 64
        q = (r.standard_normal((b, d)) * (1 + seed)).astype(np.float32)
        k = (r.standard_normal((b, d)) * 0.7 + 0.2).astype(np.float32)
        qh, kh = mxfp4.quantise(q)[2], mxfp4.quantise(k)[2]
        err = (qh @ kh.T - q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
        qm, km = T.block_moments(q, b), T.block_moments(k, b)
        sk2 = (2.0 * T.MXFP4_U ** 2 / 3.0) * float(qm["tot_m2"][0]) * float(km["tot_m2"][0]) / d ** 2
        ratio = float((err ** 2).mean()) / sk2
        assert 1.0 / 3.0 <= ratio <= 1.0, (seed, ratio)
        verr = math.sqrt(float(((kh - k.astype(np.float64)) ** 2).sum(axis=1).mean()))
        vmod = T.MXFP4_U * math.sqrt(float(km["tot_m2"][0]) / 3.0)
        assert vmod / 3.0 <= verr <= vmod, (seed, verr, vmod)


def _rank4(t):
    """Work order of the four tiers: SKIP < SKIM < LOW < FULL."""
    return np.array([0, 2, 3, 1], np.int64)[np.asarray(t, np.int64)]


def test_price_rule_structure_four_tiers():
    """With the SKIM tier: its predicted error lies above LOW's (a coarser
    format) and below SKIP's where skipping is costly; every tile takes the
    minimum of its four objectives; raising the price never moves a tile to a
    more costly tier; price 0 gives FULL, a prohibitive price SKIP; ties go
    to the cheaper tier."""
    r = np.random.default_rng(7)
    n, d, bq, bk = 512, 32, 64, 32
    q, k = [r.standard_normal((n, d)).astype(np.float32) for _ in range(2)]
    # values sharing a mean direction: skipping loses the mass deficit on a
    # large mean, while MXFP4's value error stays near LOW's, so SKIM pays for
    # some tiles (with zero-mean values LOW dominates it everywhere)
    v = (r.standard_normal((n, d)) * 0.3 + 3.0 * r.standard_normal((1, d))).astype(np.float32)
    c = cfg(bq, bk, 0.0)
    c.tau_skim = 1e-4
    base = T.oracle_plan(q, k, v, c)
    info, p = base["price"], base["price"]["pt"]
    assert info["eK"] is not None and np.all(info["eK"] >= info["eL"])
    seen = set()
    prev = None
    for lam in [0.0] + np.logspace(-5, 1, 61).tolist() + [1e3]:
        t, objs = T.tiers_price(p, info["eS"], info["eL"], lam, bk, eK=info["eK"])
        oS, oL, oF, oK = objs
        by_tier = np.stack([oS, oL, oF, oK])          # indexed by tier byte
        assert np.all(np.take_along_axis(by_tier, np.asarray(t, np.int64)[None], 0)[0] == by_tier.min(axis=0))
        if prev is not None:
            assert np.all(_rank4(t) <= _rank4(prev))
        prev = t
        seen |= set(np.unique(t).tolist())
        if lam == 0.0:
            assert np.all(t[(p * info["eS"] > 0) & (p * info["eK"] > 0)] == FULL)
        if lam == 1e3:
            assert np.all(t == SKIP)
    assert T.SKIM in seen, seen
    z = np.zeros((1, 3))
    t, _ = T.tiers_price(z, z, z, 0.0, bk, eK=z)
    assert np.all(t == SKIP)
    # a SKIM/LOW tie at equal objectives goes to SKIM (the cheaper)
    # (p = 1, price 1: SKIM 0.25 + 0.375 = LOW 0.125 + 0.5 = 0.625 < FULL 1 < SKIP)
    t, _ = T.tiers_price(np.ones((1, 1)), np.full((1, 1), 10.0), np.full((1, 1), 0.125),
                         1.0, bk, eK=np.full((1, 1), 0.25))
    assert t[0, 0] == T.SKIM
