"""Pins of the attention oracle to closed forms, identities and hand-worked
examples (P1, P2, P3, P5, P7, P8, the fp8 error bound, and the low tier's
quantised probabilities against a hand-worked tile and a scalar-loop
recomputation)."""
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
                               rows=rows, mx4=plan.get("mx4"))


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


def test_p7_degenerate_low_tile_equals_full():
    """Q, K, V on the e4m3 grid with block amax 448 (scale exactly 1) and equal
    scores inside every tile (pi == 1): the LOW partial is the FULL partial."""
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
    # q's block amax must be 448 for an exact scale: scale q up
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
    t_low = np.full((nq, nk), LOW, np.uint8)
    t_full = np.full((nq, nk), FULL, np.uint8)
    o_low = fwd(q, k, v, plan_l, c, tiers=t_low)
    o_full = fwd(q, k, v, plan_l, c, tiers=t_full)
    assert np.max(np.abs(o_low - o_full)) < 1e-12


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


def test_dequantise_rounds_once_to_fp32():
    """The low tier's value operand is decode(code) * scale rounded once to
    float32: within half a float32 ulp of the exact product, and exact when
    the scale is a power of two (the code values have 4 significant bits)."""
    r = np.random.default_rng(8)
    codes = r.integers(0, 256, size=(64 * 3, 8)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    sv = (r.uniform(0.001, 0.05, size=3)).astype(np.float32)
    got = T.dequantise(codes, sv, 64)
    exact = T.e4m3.decode(codes) * np.repeat(sv.astype(np.float64), 64)[:, None]
    tol = np.abs(exact) * 2.0 ** -24
    assert np.all(np.abs(got - exact) <= tol * 1.0000001)
    assert not np.array_equal(got, exact)             # the rounding happens
    p2 = np.array([2.0 ** -7, 2.0 ** -3, 1.0], np.float32)
    assert np.array_equal(T.dequantise(codes, p2, 64), T.e4m3.decode(codes) * np.repeat(p2.astype(np.float64), 64)[:, None])


def test_low_hand_example():
    """A hand-worked LOW tile (tests/golden/low_hand_example.txt): the codes of
    its probabilities and the merged output."""
    g = _read("low_hand_example.txt")
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    v = np.array(g["v"], np.float32)
    c = cfg(2, 2)
    t = np.array([[FULL, LOW], [LOW, FULL]], np.uint8)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    assert plan["sq"][0] == np.float32(2.0 ** -8) and plan["sk"][1] == np.float32(2.0 ** -8)
    s = T.low_scores(T.e4m3.decode(plan["q8"][0:2]), plan["sq"][0], T.e4m3.decode(plan["k8"][2:4]),
                     plan["sk"][1], 4)
    _, _, codes, _ = T.quantised_probabilities(s)
    assert codes[0].tolist() == [int(x) for x in g["codes01_row0"][0]]
    o = fwd(q, k, v, plan, c)
    assert abs(o[0, 0] - g["O0"][0][0]) < 1e-12


def _scalar_e4m3():
    import importlib.util
    spec = importlib.util.spec_from_file_location("e4m3pins", os.path.join(os.path.dirname(__file__),
                                                                           "test_oracle_e4m3.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod._bitwise_rne_e4m3


@pytest.mark.parametrize("n,d,bq,bk", [(96, 16, 32, 16), (70, 8, 32, 32)])
def test_low_partials_against_scalar_loops(n, d, bq, bk):
    """Every LOW tile's partial (m_t, sum pi, sum pi v^) against explicit loops:
    scores summed term by term from the decoded codes, the tile maximum, x =
    float32(448 e^{s - m_t}) encoded by the bitwise E4M3 encoder of the codec
    pins, values decode(code) * scale rounded to float32."""
    import struct
    enc = _scalar_e4m3()
    q, k, v = rand_qkv(n, d, 31 + n, scale=1.4)
    c = cfg(bq, bk)
    nq, nk = -(-n // bq), -(-n // bk)
    t = np.full((nq, nk), LOW, np.uint8)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    t = plan["tiers"]
    _, parts = T.attention_forward(q, k, v, t, bq, bk, plan["kbar"], plan["vbar"], plan["q8"], plan["sq"],
                                   plan["k8"], plan["sk"], plan["v8"], plan["sv"], return_partials=True)
    dec = T.e4m3.DECODE
    f32 = lambda x: struct.unpack("<f", struct.pack("<f", x))[0]
    for I in range(nq):
        ms, ls, os_, _, _, _ = parts[I]
        lows = [J for J in range(nk) if t[I, J] == LOW]
        if not lows:
            continue
        m_low, l_low, o_low = ms[-1], ls[-1], os_[-1]             # LOW is the last kept group here
        for a, J in enumerate(lows):
            keys = range(J * bk, min(n, (J + 1) * bk))
            for ii, i in enumerate(range(I * bq, min(n, (I + 1) * bq))):
                s = []
                for j in keys:
                    acc = 0.0
                    for x in range(d):
                        acc += dec[plan["q8"][i, x]] * dec[plan["k8"][j, x]]
                    s.append(acc * float(plan["sq"][I]) * float(plan["sk"][J]) / math.sqrt(d))
                mt = max(s)
                pis = [dec[enc(f32(448.0 * math.exp(sj - mt)))] / 448.0 for sj in s]
                assert max(pis) == 1.0                               # the maximum lands on 448
                vh = [[f32(dec[plan["v8"][j, x]] * float(plan["sv"][J])) for x in range(d)] for j in keys]
                assert abs(m_low[ii, a] - mt) <= 1e-12 * max(1.0, abs(mt))
                assert abs(l_low[ii, a] - sum(pis)) <= 1e-12
                ov = [sum(p * vh[jj][x] for jj, p in enumerate(pis)) for x in range(d)]
                assert np.max(np.abs(o_low[ii, a] - np.array(ov))) <= 1e-12


def test_quantised_probabilities_structure():
    """Codes of a quantised tile: the maximum is code 0x7E (448) in every row,
    codes are monotone in the scores, keys past the sequence end get code 0,
    and each x lies within half an E4M3 step of its code's value."""
    r = np.random.default_rng(12)
    s = r.standard_normal((40, 64)) * 3.0
    s[:, 50:] = -np.inf
    mt, x, c, pi = T.quantised_probabilities(s)
    assert np.all(c.max(axis=1) == 0x7E) and np.all(pi.max(axis=1) == 1.0)
    assert np.all(c[:, 50:] == 0) and np.all(pi[:, 50:] == 0)
    for row in range(40):
        o = np.argsort(s[row, :50])
        assert np.all(np.diff(c[row, :50][o].astype(int)) >= 0)
    val = T.e4m3.decode(c)
    # half a step: 2^-4 relative for normals (>= 2^-6), 2^-10 absolute below
    tol = np.maximum(np.abs(val) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(x - val) <= tol * 1.0000001)


def test_p_codes_override():
    """Given its own codes the forward is unchanged; a code moved to the
    neighbouring E4M3 value changes only that tile's row."""
    n, d, bq, bk = 128, 16, 32, 32
    q, k, v = rand_qkv(n, d, 41, scale=1.3)
    c = cfg(bq, bk)
    t = np.full((4, 4), LOW, np.uint8)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    t = plan["tiers"]
    o = fwd(q, k, v, plan, c)
    s = T.low_scores(T.e4m3.decode(plan["q8"][0:32]), plan["sq"][0], T.e4m3.decode(plan["k8"][64:96]),
                     plan["sk"][2], d)
    codes = T.quantised_probabilities(s)[2]
    o_same = T.oracle_forward(q, k, v, plan, bq, bk, p_codes={(0, 2): codes})
    assert np.array_equal(o, o_same)
    alt = codes.copy()
    j = int(np.argmax(codes[5] < 0x7E))
    alt[5, j] += 1
    o_alt = T.oracle_forward(q, k, v, plan, bq, bk, p_codes={(0, 2): alt})
    diff = np.abs(o_alt - o).max(axis=1)
    assert diff[5] > 0 and np.all(diff[np.arange(n) != 5] == 0)
