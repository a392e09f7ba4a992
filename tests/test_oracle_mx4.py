"""Pins of the oracle's skim tier: the MXFP4 codec against the format's
definition (OCP Microscaling Formats v1.0: E2M1 elements, E8M0 block scale of
32 elements), the four-tier threshold map and lists, and the skim tile inside
the single-pass forward (exact on representable inputs; brute force against
the dense weight matrix on tiny inputs)."""
import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import FULL, LOW, SKIM, SKIP, mxfp4
from oracle import tattn as T


def _e2m1_from_fields(c):
    """Value of a 4-bit code from its bit fields: sign, 2-bit exponent (bias 1),
    1 mantissa bit; exponent field 0 is subnormal (m * 0.5 * 2^0)."""
    s = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    return s * (m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))


def test_decode_matches_bit_fields():
    for c in range(16):
        assert mxfp4.decode(np.array([c]))[0] == _e2m1_from_fields(c)
    assert mxfp4.decode(np.array([7]))[0] == 6.0 and mxfp4.decode(np.array([1]))[0] == 0.5


def test_encode_grid_midpoints_saturation_sign():
    grid = np.array([_e2m1_from_fields(c) for c in range(8)])
    assert np.array_equal(mxfp4.decode(mxfp4.encode(grid)), grid)
    assert np.array_equal(mxfp4.decode(mxfp4.encode(-grid[1:])), -grid[1:])
    # each midpoint goes to the neighbour whose mantissa bit is 0
    mids = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in mids.items():
        assert mxfp4.decode(mxfp4.encode(np.array([x])))[0] == want, x
        assert mxfp4.decode(mxfp4.encode(np.array([-x])))[0] == -want, x
    # off the midpoints: nearest
    for x, want in {0.2499: 0.0, 0.2501: 0.5, 4.99: 4.0, 5.01: 6.0, 2.49: 2.0, 2.51: 3.0}.items():
        assert mxfp4.decode(mxfp4.encode(np.array([x])))[0] == want, x
    # saturation and signed zero
    assert np.all(mxfp4.decode(mxfp4.encode(np.array([6.5, 7.99, 1e30]))) == 6.0)
    assert mxfp4.encode(np.array([-0.1]))[0] == 8 and mxfp4.encode(np.array([0.1]))[0] == 0


def test_encode_equals_stepwise_rounding():
    """A second formulation of round-to-nearest-even on the E2M1 grid: spacing
    0.5 below 2, 1 in [2, 4), 2 in [4, 8), then clamp to 6."""
    r = np.random.default_rng(3)
    a = np.concatenate([r.uniform(0, 8, 20000), np.arange(0, 8.01, 0.125), r.uniform(0, 0.3, 2000)])
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    q = np.minimum(np.rint(a / step) * step, 6.0)
    assert np.array_equal(mxfp4.decode(mxfp4.encode(a)), q)


def test_block_exponent_closed_form():
    r = np.random.default_rng(4)
    for _ in range(200):
        k = int(r.integers(-120, 120))
        amax = (1.0 + r.uniform(0, 1)) * 2.0 ** k          # in [2^k, 2^(k+1))
        x = r.uniform(-1, 1, 32) * amax
        x[int(r.integers(32))] = -amax
        assert mxfp4.block_exponents(x[None])[0, 0] == k - 2
    assert mxfp4.block_exponents(np.zeros((1, 32)))[0, 0] == -127
    assert mxfp4.block_exponents(np.full((1, 32), 2.0 ** -130))[0, 0] == -127     # clamped
    assert mxfp4.block_exponents(np.full((1, 32), 2.0 ** 127))[0, 0] == 125


def test_quantise_round_trips_representable_blocks():
    r = np.random.default_rng(5)
    grid = mxfp4.decode(np.arange(16))
    for _ in range(50):
        e = r.integers(-20, 20, size=(3, 4))
        y = r.choice(grid, size=(3, 4, 32))
        y[..., 0] = r.choice([4.0, -4.0, 6.0, -6.0], size=(3, 4))    # amax in [4, 8) * 2^e
        x = np.ldexp(y, e[..., None]).reshape(3, 128)
        codes, sb, deq = mxfp4.quantise(x)
        assert np.array_equal(deq, x)
        assert np.array_equal(sb.astype(np.int64) - 127, e)
        assert np.array_equal(mxfp4.decode(codes), y.reshape(3, 128))


def test_quantise_error_bound():
    """|x - deq| <= half the grid spacing at x / 2^e, times 2^e; above 6 the
    clamp error is below 2 * 2^e."""
    r = np.random.default_rng(6)
    x = r.standard_normal((64, 128)) * np.exp(r.uniform(-5, 5, (64, 1)))
    _, sb, deq = mxfp4.quantise(x)
    e = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(np.ldexp(x, -e))
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, np.where(y <= 6, 1.0, 2.0)))
    assert np.all(np.abs(x - deq) <= np.ldexp(half, e))
    assert np.all(y < 8)


def test_pack_nibbles_order():
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(mxfp4.pack_nibbles(c), [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE])


def test_four_tier_thresholds_and_lists():
    p = np.array([[0.5, 0.02, 0.005, 5e-4, 1e-5, 2e-4]])
    t = T.tiers_threshold(p, 0.1, 0.001, tau_skim=1e-4)
    assert t.tolist() == [[FULL, LOW, LOW, SKIM, SKIP, SKIM]]
    assert T.tiers_threshold(p, 0.1, 0.001).tolist() == [[FULL, LOW, LOW, SKIP, SKIP, SKIP]]
    assert T.tiers_threshold(p, 0.1, 0.001, top_k=3, tau_skim=1e-4).tolist() == [[FULL, LOW, LOW, SKIP, SKIP, SKIP]]
    assert T.tiers_threshold(p, 0.1, 0.001, top_k=4, tau_skim=1e-4).tolist() == [[FULL, LOW, LOW, SKIM, SKIP, SKIP]]
    lists, counts = T.build_lists(t)
    assert lists.tolist() == [[0, 1, 2, 3, 5, 4]] and counts.tolist() == [[1, 2, 1]]


def _representable(r, n, d, lo=-6, hi=6):
    """Rows whose 32-blocks are E2M1 values times 2^e with an element of
    magnitude 4 or 6, so MXFP4 keeps them exactly."""
    grid = mxfp4.decode(np.arange(16))
    y = r.choice(grid, size=(n, d // 32, 32))
    y[..., 0] = r.choice([4.0, -4.0, 6.0, -6.0], size=(n, d // 32))
    e = r.integers(lo, hi, size=(n, d // 32, 1))
    return np.ldexp(y, e).reshape(n, d).astype(np.float32)


def _plan_and_fwd(q, k, v, bq, bk, t):
    c = SimpleNamespace(block_q=bq, block_k=bk, tau_hi=0.05, tau_lo=0.005, top_k=0, mode=3,
                        keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=t)
    o = T.attention_forward(q, k, v, t, bq, bk, plan["kbar"], plan["vbar"], plan["q8"], plan["sq"],
                            plan["k8"], plan["sk"], plan["v8"], plan["sv"], mx4=plan["mx4"])
    return plan, o


def test_skim_scores_on_representable_inputs_are_exact():
    """On inputs MXFP4 keeps exactly, a SKIM tile's scores are the exact
    scores: its partial equals the low tier's quantised-probability partial
    (codes against the tile maximum, E4M3 values) computed here from the
    unquantised q and k, tile by tile.  (The forward runs the map as given,
    diagonal tiles included.)"""
    r = np.random.default_rng(7)
    n, d, bq, bk = 200, 64, 64, 16          # ragged last blocks
    q = _representable(r, n, d, -8, -4)
    k, v = _representable(r, n, d, -4, -1), _representable(r, n, d, -3, 0)
    nq, nk = -(-n // bq), -(-n // bk)
    t = np.full((nq, nk), SKIM, np.uint8)
    plan, o = _plan_and_fwd(q, k, v, bq, bk, t)
    for x, name in ((q, "q"), (k, "k")):
        assert np.array_equal(plan["mx4"][name], x.astype(np.float64))
    vh = T.dequantise(plan["v8"], plan["sv"], bk)
    isd = 1.0 / np.sqrt(d)
    for i in range(0, n, 7):
        I = i // bq
        refs, nums, dens = [], [], []
        for J in range(nk):
            j0, j1 = J * bk, min(n, (J + 1) * bk)
            s = (k[j0:j1].astype(np.float64) @ q[i].astype(np.float64)) * isd
            if t[I, J] == FULL:
                m = s.max()
                e = np.exp(s - m)
                refs.append(m); dens.append(e.sum()); nums.append(e @ v[j0:j1].astype(np.float64))
            else:
                m, _, _, pi = T.quantised_probabilities(s)
                refs.append(m); dens.append(pi.sum()); nums.append(pi @ vh[j0:j1])
        M = max(refs)
        w = np.exp(np.array(refs) - M)
        ref = (w[:, None] * np.array(nums)).sum(0) / (w * np.array(dens)).sum()
        assert np.max(np.abs(o[i] - ref)) < 1e-12, i


def test_skim_differs_from_full_on_general_inputs():
    """A skim tile must run on the 4-bit copies, not the inputs."""
    r = np.random.default_rng(8)
    n, d, bq, bk = 128, 64, 64, 64
    q, k, v = [r.standard_normal((n, d)).astype(np.float32) for _ in range(3)]
    _, o_k = _plan_and_fwd(q, k, v, bq, bk, np.full((2, 2), SKIM, np.uint8))
    _, o_f = _plan_and_fwd(q, k, v, bq, bk, np.full((2, 2), FULL, np.uint8))
    err = np.abs(o_k - o_f)
    assert err.max() > 1e-3 and err.mean() < 0.2


def test_four_tier_forward_equals_dense_weights():
    r = np.random.default_rng(9)
    n, d, bq, bk = 96, 32, 32, 16
    q, k, v = [(r.standard_normal((n, d)) * 1.2).astype(np.float32) for _ in range(3)]
    nq, nk = n // bq, n // bk
    t = r.integers(0, 4, (nq, nk)).astype(np.uint8)
    plan, o = _plan_and_fwd(q, k, v, bq, bk, t)
    assert np.any(t == SKIM) and np.any(t == SKIP) and np.any(t == LOW)
    W, vsel = T.effective_weights(q, k, v, t, bq, bk, plan["kbar"], plan["q8"], plan["sq"], plan["k8"],
                                  plan["sk"], plan["v8"], plan["sv"], mx4=plan["mx4"])
    assert np.max(np.abs(W.sum(axis=1) - 1)) < 1e-12
    o_w = np.einsum("ij,ijd->id", W, vsel)
    # the forward values skipped tiles with the float32-stored block means
    assert np.max(np.abs(o - o_w)) < 2.0 ** -24 * np.abs(v).max() * 2
