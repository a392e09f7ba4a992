"""Pins of the attention oracle to closed forms, identities and hand-worked
examples (P1, P2, P3, P5, P7, P8 and the fp8 error bound)."""
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from oracle import FULL, LOW, SKIP
from oracle import tattn as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def cfg(bq, bk, tau_hi=0.05, tau_lo=0.005, top_k=0, mode=0):
    return SimpleNamespace(block_q=bq, block_k=bk, tau_hi=tau_hi, tau_lo=tau_lo, top_k=top_k,
                           mode=mode, keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256)


def rand_qkv(n, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return [(r.standard_normal((n, d)) * scale).astype(np.float32) for _ in range(3)]


def fwd(q, k, v, plan, c, tiers=None, rows=None):
    t = plan["tiers"] if tiers is None else tiers
    return T.attention_forward(q, k, v, t, c.block_q, c.block_k, plan["kbar"], plan["vbar"],
                               plan["q8"], plan["sq"], plan["k8"], plan["sk"], plan["v8"], plan["sv"],
                               rows=rows)


def _read(name):
    rows = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        rows.setdefault(key, []).append([float(x) for x in vals])
    return rows


def test_router_hand_example():
    g = _read("router_hand_example.txt")
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    qbar, kbar = T.pool_means(q, 2), T.pool_means(k, 2)
    _, p = T.router(qbar, kbar, 3, 2)
    for key in ("p00", "p01", "p10", "p11"):
        i, j = int(key[1]), int(key[2])
        assert abs(p[i, j] - g[key][0][0]) < 1e-15


def test_skip_hand_example():
    g = _read("skip_hand_example.txt")
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    v = np.array(g["v"], np.float32)
    c = cfg(2, 2)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=np.array([[FULL, SKIP], [SKIP, FULL]], np.uint8))
    o = fwd(q, k, v, plan, c)
    assert abs(o[0, 0] - g["O0"][0][0]) < 1e-14


@pytest.mark.parametrize("n,d,bq,bk", [(256, 64, 64, 64), (200, 16, 64, 32), (130, 8, 32, 64), (77, 4, 16, 16)])
def test_p1_all_full_equals_naive(n, d, bq, bk):
    q, k, v = rand_qkv(n, d, n + d)
    c = cfg(bq, bk)
    plan = T.oracle_plan(q, k, v, c, mode=2)
    assert np.all(plan["tiers"] == FULL)
    o = fwd(q, k, v, plan, c)
    ref = T.naive_attention(q, k, v)
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("n,d,bq,bk", [(256, 32, 64, 64), (250, 16, 64, 16), (97, 8, 32, 64), (300, 16, 128, 64)])
def test_p2_constant_keys_skip_is_exact(n, d, bq, bk):
    r = np.random.default_rng(n * 7 + d)
    nk = -(-n // bk)
    cent = r.standard_normal((nk, d)).astype(np.float32) * 2
    k = np.repeat(cent, bk, axis=0)[:n]
    q = r.standard_normal((n, d)).astype(np.float32)
    v = r.standard_normal((n, d)).astype(np.float32)
    c = cfg(bq, bk, tau_hi=2.0, tau_lo=2.0)        # every non-diagonal tile below tau_lo
    plan = T.oracle_plan(q, k, v, c)
    diag = T.diagonal_mask(n, bq, bk)
    assert np.all(plan["tiers"][~diag] == SKIP) and np.all(plan["tiers"][diag] == FULL)
    o = fwd(q, k, v, plan, c)
    ref = T.naive_attention(q, k, v)
    # exact identity up to the float32 storage of the block means vbar:
    # |error| <= 2^-24 * max|v| per element (k is constant, so kbar is exact)
    assert np.max(np.abs(o - ref)) < 2.0 ** -24 * np.abs(v).max() * 2


@pytest.mark.parametrize("mode", ["threshold", "all_low", "all_skip", "mixed", "adaptive"])
def test_p3_unit_values_give_unit_output(mode):
    n, d, bq, bk = 300, 32, 64, 32
    q, k, _ = rand_qkv(n, d, 3, scale=1.5)
    v = np.ones((n, d), np.float32)
    c = cfg(bq, bk, tau_hi=0.2, tau_lo=0.02)
    nq, nk = -(-n // bq), -(-n // bk)
    rr = np.random.default_rng(5)
    ext = {"all_low": np.full((nq, nk), LOW, np.uint8), "all_skip": np.full((nq, nk), SKIP, np.uint8),
           "mixed": rr.integers(0, 3, (nq, nk)).astype(np.uint8)}
    if mode == "threshold":
        plan = T.oracle_plan(q, k, v, c, mode=0)
    elif mode == "adaptive":
        plan = T.oracle_plan(q, k, v, c, mode=1)
    else:
        plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=ext[mode])
    o = fwd(q, k, v, plan, c)
    assert np.max(np.abs(o - 1.0)) < 1e-6


def test_p3_weights_nonnegative_and_sum_to_one():
    n, d, bq, bk = 128, 16, 32, 16
    q, k, v = rand_qkv(n, d, 11, scale=1.3)
    c = cfg(bq, bk)
    nq, nk = n // bq, n // bk
    t = np.random.default_rng(2).integers(0, 3, (nq, nk)).astype(np.uint8)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    W, vsel = T.effective_weights(q, k, v, plan["tiers"], bq, bk, plan["kbar"], plan["q8"], plan["sq"],
                                  plan["k8"], plan["sk"], plan["v8"], plan["sv"])
    assert W.min() >= 0
    assert np.max(np.abs(W.sum(axis=1) - 1)) < 1e-12
    o_w = np.einsum("ij,ijd->id", W, vsel)
    o = fwd(q, k, v, plan, c)
    # the forward values skipped tiles with the float32-stored vbar; W uses exact v
    assert np.max(np.abs(o - o_w)) < 2.0 ** -24 * np.abs(v).max() * 2


@pytest.mark.parametrize("n,bq,bk", [(256, 64, 64), (250, 64, 16), (190, 32, 64)])
def test_p5_constant_blocks_give_exact_block_mass(n, bq, bk):
    d = 16
    r = np.random.default_rng(n)
    nq, nk = -(-n // bq), -(-n // bk)
    q = np.repeat(r.standard_normal((nq, d)), bq, axis=0)[:n].astype(np.float32)
    k = np.repeat(r.standard_normal((nk, d)), bk, axis=0)[:n].astype(np.float32)
    qbar, kbar = T.pool_means(q, bq), T.pool_means(k, bk)
    _, p = T.router(qbar, kbar, n, bk)
    s = q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    for I in range(nq):
        i = I * bq
        mass = np.array([w[i, J * bk:(J + 1) * bk].sum() for J in range(nk)])
        assert np.max(np.abs(p[I] - mass) / mass) < 1e-12


def _nearest_e4m3(y):
    """Nearest E4M3 value by brute force over the 127 non-negative finite
    values, ties to the even code (an independent formulation of the
    format's rounding, for non-negative y below 448)."""
    grid = T.e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    dist = np.abs(grid - y)
    best = np.flatnonzero(dist == dist.min())
    return grid[best[0]] if best.size == 1 else grid[best[best % 2 == 0][0]]


def test_p7_degenerate_low_tiles_closed_form():
    """Q, K, V on the e4m3 grid with block amax 448 (K and V scale exactly 1)
    and equal scores inside every tile: every LOW tile J of a row acts as one
    score s_J, so O_i = sum_J n_J w_J v_J / sum_J n_J w_J with v_J the block's
    value mean and w_J = 2^t rounded to E4M3 on the tile's reference,
    t = s_J log2(e): w_J = nearest(2^(t - ceil(t) + 8)) 2^(ceil(t) - 8).  With
    every tile FULL the same holds with w_J = e^(s_J)."""
    n, d, bq, bk = 128, 16, 32, 32
    r = np.random.default_rng(9)
    grid = T.e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    grid = np.concatenate([grid, -grid])
    nk = n // bk
    kc = r.choice(grid[np.abs(grid) <= 8], size=(nk, d))
    kc[:, 0] = 448.0
    k = np.repeat(kc, bk, axis=0).astype(np.float32)
    q = r.choice(grid[np.abs(grid) <= 2], size=(n, d)).astype(np.float32) * 1e-3
    q = T.e4m3.decode(T.e4m3.encode(q)).astype(np.float32)
    q[::bq, 1] = 448.0 * 1e-3
    q = T.e4m3.decode(T.e4m3.encode(q)).astype(np.float32)
    for I in range(n // bq):
        blk = q[I * bq:(I + 1) * bq]
        q[I * bq:(I + 1) * bq] = blk * np.float32(448.0 / np.abs(blk).max())
    q = T.e4m3.decode(T.e4m3.encode(q)).astype(np.float32)
    q *= np.float32(1.0 / 4096)   # keep scores modest; divides amax by a power of two
    v = r.choice(grid[np.abs(grid) <= 64], size=(n, d)).astype(np.float32)
    v[::bk, 0] = 448.0
    c = cfg(bq, bk)
    nq = n // bq
    plan_l = T.oracle_plan(q, k, v, c, mode=3, external_tiers=np.full((nq, nk), LOW, np.uint8))
    assert np.all(plan_l["sk"] == 1) and np.all(plan_l["sv"] == 1)
    assert np.all(plan_l["sq"] == np.float32(1.0 / 4096))
    o_low = fwd(q, k, v, plan_l, c, tiers=np.full((nq, nk), LOW, np.uint8))
    o_full = fwd(q, k, v, plan_l, c, tiers=np.full((nq, nk), FULL, np.uint8))
    vbar = v.astype(np.float64).reshape(nk, bk, d).mean(axis=1)
    S = q.astype(np.float64) @ kc.T / np.sqrt(d)                       # [n, Nk]
    rounded = 0
    for i in range(n):
        t = S[i] / np.log(2.0)
        ref = np.ceil(t)
        w_low = np.array([_nearest_e4m3(2.0 ** (tj - rj + 8)) * 2.0 ** (rj - 8) for tj, rj in zip(t, ref)])
        w_full = np.exp(S[i])
        rounded += np.sum(np.abs(w_low / 2.0 ** t - 1) > 1e-9)
        for w, o in ((w_low, o_low), (w_full, o_full)):
            want = (w[:, None] * vbar).sum(axis=0) / w.sum()
            assert np.max(np.abs(o[i] - want)) < 1e-12, i
    assert rounded > 0.5 * n * nk      # the rounding is real, not a no-op


def test_p8_permuting_keys_inside_blocks_is_invariant():
    n, d, bq, bk = 256, 16, 64, 32
    q, k, v = rand_qkv(n, d, 21, scale=1.2)
    _, p0 = T.router(T.pool_means(q, bq), T.pool_means(k, bk), n, bk)
    c = cfg(bq, bk, tau_hi=float(np.quantile(p0, 0.8)), tau_lo=float(np.quantile(p0, 0.3)))
    plan = T.oracle_plan(q, k, v, c)
    assert set(np.unique(plan["tiers"])) == {SKIP, LOW, FULL}
    o = fwd(q, k, v, plan, c)
    perm = np.arange(n)
    r = np.random.default_rng(4)
    for J in range(n // bk):
        perm[J * bk:(J + 1) * bk] = r.permutation(perm[J * bk:(J + 1) * bk])
    kp, vp = k[perm], v[perm]
    plan_p = T.oracle_plan(q, kp, vp, c)
    assert np.array_equal(plan_p["tiers"], plan["tiers"])
    o_p = fwd(q, kp, vp, plan_p, c)
    assert np.max(np.abs(o - o_p)) < 1e-12


def test_p8_lower_tau_hi_never_demotes():
    r = np.random.default_rng(1)
    p = r.dirichlet(np.ones(64) * 0.3, size=16)
    t1 = T.tiers_threshold(p, 0.05, 0.005)
    t2 = T.tiers_threshold(p, 0.02, 0.005)
    assert np.all(t2 >= t1)


def test_low_tier_within_fp8_error_of_exact():
    """Every tile LOW: the result stays within the e4m3 rounding budget of exact
    attention (3 mantissa bits: relative step 1/8, half-step 1/16 per operand)."""
    n, d, bq, bk = 256, 64, 64, 64
    q, k, v = rand_qkv(n, d, 13)
    c = cfg(bq, bk)
    nq, nk = n // bq, n // bk
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=np.full((nq, nk), LOW, np.uint8))
    t = np.full((nq, nk), LOW, np.uint8)
    o = fwd(q, k, v, plan, c, tiers=t)
    ref = T.naive_attention(q, k, v)
    err = np.abs(o - ref)
    # each v^ is within half an e4m3 step (1/16 relative) of v and each weight
    # within ~1/16 plus the score error; these errors average over the keys, so
    # the output error sits far below max|v|/16 ~ 0.25.  A dropped scale or a
    # missing 1/448 gives errors of order 1 or more.
    assert err.max() < 0.1 and err.mean() < 0.005
    # and a gross mistake (e.g. forgetting the value scale) would be far outside it
    assert np.max(np.abs(ref)) > 0.1


def test_lists_partition_and_order():
    r = np.random.default_rng(3)
    t = r.integers(0, 3, (10, 37)).astype(np.uint8)
    lists, counts = T.build_lists(t)
    for i in range(10):
        nf, nl, ns = counts[i]
        assert nf + nl + ns == 37
        assert sorted(lists[i].tolist()) == list(range(37))
        f, lo, s = lists[i][:nf], lists[i][nf:nf + nl], lists[i][nf + nl:]
        assert np.all(np.diff(f) > 0) and np.all(np.diff(lo) > 0) and np.all(np.diff(s) > 0)
        assert np.all(t[i, f] == FULL) and np.all(t[i, lo] == LOW) and np.all(t[i, s] == SKIP)


def test_value_exponents_closed_form():
    """The power-of-two V scale 2^e is the smallest with amax <= 448 * 2^e:
    amax in (448 * 2^(e-1), 448 * 2^e] gives e; an all-zero block gives 0;
    the codes then dequantise exactly to within half an E4M3 step."""
    r = np.random.default_rng(8)
    for e in list(range(-20, 21)) + [-126, 100]:
        for amax in (448.0 * 2.0 ** e, np.nextafter(448.0 * 2.0 ** e, 0), 448.0 * 2.0 ** (e - 1) * 1.0000001,
                     448.0 * 2.0 ** e * r.uniform(0.51, 0.99)):
            x = np.zeros((64, 4), np.float64)
            x[5, 2] = -amax
            x[7] = r.uniform(-1, 1, 4) * amax
            got = T.value_exponents(x, 64)[0]
            assert got == e, (e, amax, got)
    assert T.value_exponents(np.zeros((64, 4)), 64)[0] == 0
    v = (r.standard_normal((3 * 64, 8)) * np.array([1e-3, 1.0, 300.0]).repeat(64)[:, None]).astype(np.float32)
    codes, sv, ev = T.quantise_values(v, 64)
    assert np.array_equal(sv.astype(np.float64), 2.0 ** ev)
    vh = T.low_values(codes, sv, 64)
    assert np.array_equal(vh, T.e4m3.decode(codes) * np.repeat(2.0 ** ev, 64)[:, None])
    # RNE on 3 mantissa bits: |v - v^| <= 2^-4 |v| above the subnormal range
    big = np.abs(v) >= np.repeat(2.0 ** (ev - 6), 64)[:, None]
    assert np.all(np.abs(v - vh)[big] <= 2.0 ** -4 * np.abs(v)[big] * (1 + 1e-12))
    for j in range(3):
        blk = np.abs(v[64 * j:64 * (j + 1)]).max()
        assert 224.0 < blk / sv[j] <= 448.0


def test_low_weights_within_half_step_of_exact():
    """Every tile LOW on tiny inputs: each low weight is the exact softmax
    weight of the fp8 scores times a factor in [1 - 1/16, 1 + 1/16] (E4M3
    keeps 3 mantissa bits; codes below 2^-6 are excluded), up to the common
    normalisation, and the quantisation does move the weights."""
    n, d, bq, bk = 96, 32, 32, 32
    q, k, v = rand_qkv(n, d, 17, scale=1.5)
    c = cfg(bq, bk)
    nq, nk = n // bq, n // bk
    t = np.full((nq, nk), LOW, np.uint8)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    W, _ = T.effective_weights(q, k, v, t, bq, bk, plan["kbar"], plan["q8"], plan["sq"], plan["k8"],
                               plan["sk"], plan["v8"], plan["sv"])
    qh = T.e4m3.decode(plan["q8"]) * np.repeat(plan["sq"].astype(np.float64), bq)[:, None]
    kh = T.e4m3.decode(plan["k8"]) * np.repeat(plan["sk"].astype(np.float64), bk)[:, None]
    S = qh @ kh.T / np.sqrt(d)
    Wx = np.exp(S - S.max(axis=1, keepdims=True))
    Wx /= Wx.sum(axis=1, keepdims=True)
    ratio = W / Wx
    # the tile reference: codes below 2^-6 are subnormal and coarser
    t2 = S / np.log(2.0)
    ref = np.ceil(t2.reshape(n, nk, bk).max(axis=2)).repeat(bk, axis=1)
    normal = 2.0 ** (t2 - ref + 8) >= 2.0 ** -6
    lo, hi = (15 / 16) / (17 / 16), (17 / 16) / (15 / 16)
    assert np.all((ratio[normal] >= lo * (1 - 1e-12)) & (ratio[normal] <= hi * (1 + 1e-12)))
    assert np.max(np.abs(ratio - 1)) > 1e-3
    assert np.max(np.abs(W.sum(axis=1) - 1)) < 1e-12
