"""Pins of the oracle's residual-corrected refine scores (Triage: a tile
refined with 4-bit residual correction; reading R20): each operand is MXFP4
plus an MXFP4 residual, and a tile's scores keep the three products of order
up to one in the residuals."""
from types import SimpleNamespace

import numpy as np

from oracle import FULL, LOW, SKIM, mxfp4
from oracle import tattn as T


def _grid_rows(r, n, d, e, lead=(6.0, -6.0)):
    """Rows whose 32-blocks are E2M1 values times 2^e (e per block) with a
    leading element of magnitude `lead`, so MXFP4 keeps them exactly with
    block exponent e."""
    grid = mxfp4.decode(np.arange(16))
    y = r.choice(grid, size=(n, d // 32, 32))
    y[..., 0] = r.choice(lead, size=(n, d // 32))
    return np.ldexp(y, e).reshape(n, d)


def test_residual_reconstruction_error_bound():
    """x4 + x4r approximates x to within the residual's own grid: at most
    2^(e_r + 1) per element (half the widest E2M1 spacing, or the clamp at 6),
    e_r the residual block's exponent; and far better than x4 alone."""
    r = np.random.default_rng(11)
    x = (r.standard_normal((40, 128)) * np.exp(r.standard_normal((40, 1)))).astype(np.float32)
    R = T.refine_operands(x, x)
    res = x.astype(np.float64) - R["q"]
    e_r = np.repeat(mxfp4.block_exponents(res), 32, axis=-1)
    err = np.abs(x - R["q"] - R["qr"])
    assert np.all(err <= np.ldexp(1.0, e_r + 1))
    assert err.max() < 0.25 * np.abs(res).max()
    assert np.array_equal(R["k"], R["q"]) and np.array_equal(R["kr"], R["qr"])


def test_two_level_inputs_give_exact_products_minus_the_residual_pair():
    """x = a + b with a on the MXFP4 grid at exponent e and b on it at e - 6:
    x rounds to a, its residual is b exactly, and the refine scores are exactly
    <xq, xk> - <bq, bk>: the dropped second-order term and nothing else."""
    r = np.random.default_rng(12)
    n, d = 48, 64
    e = r.integers(-3, 3, size=(n, d // 32, 1))
    aq, ak = _grid_rows(r, n, d, e), _grid_rows(r, n, d, e)
    bq, bk = _grid_rows(r, n, d, e - 6, (4.0, -4.0, 6.0, -6.0)), _grid_rows(r, n, d, e - 6, (4.0, -4.0, 6.0, -6.0))
    xq, xk = aq + bq, ak + bk
    R = T.refine_operands(xq, xk)
    assert np.array_equal(R["q"], aq) and np.array_equal(R["k"], ak)
    assert np.array_equal(R["qr"], bq) and np.array_equal(R["kr"], bk)
    s = T.refine_scores((R["q"], R["qr"]), (R["k"], R["kr"]))
    assert np.array_equal(s, xq @ xk.T - bq @ bk.T)
    assert not np.allclose(s, xq @ xk.T)            # the pair term is really dropped


def test_refine_scores_against_scalar_loops():
    r = np.random.default_rng(13)
    q4, q4r, k4, k4r = (r.standard_normal((5, 32)) for _ in range(4))
    s = T.refine_scores((q4, q4r), (k4, k4r))
    for i in range(5):
        for j in range(5):
            want = 0.0
            for c in range(32):
                want += q4[i, c] * k4[j, c] + q4[i, c] * k4r[j, c] + q4r[i, c] * k4[j, c]
            assert abs(s[i, j] - want) <= 1e-12 * (1 + abs(want))


def _cfg(bq, bk, refine):
    return SimpleNamespace(block_q=bq, block_k=bk, tau_hi=0.05, tau_lo=0.005, top_k=0, mode=3,
                           keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256, low_refine=refine)


def _fwd(q, k, v, bq, bk, t, refine):
    plan = T.oracle_plan(q, k, v, _cfg(bq, bk, refine), mode=3, external_tiers=t)
    return plan, T.oracle_forward(q, k, v, plan, bq, bk)


def test_refined_low_tiles_equal_skim_tiles_where_the_residual_vanishes():
    """On inputs MXFP4 keeps exactly the residuals are zero, so a refined LOW
    tile runs SKIM's arithmetic (same scores, same quantised probabilities and
    E4M3 values): the two forwards agree to rounding, tile map for tile map."""
    r = np.random.default_rng(14)
    n, d, bq, bk = 192, 64, 64, 64
    q = _grid_rows(r, n, d, r.integers(-8, -5, size=(n, d // 32, 1))).astype(np.float32)
    k = _grid_rows(r, n, d, r.integers(-4, -1, size=(n, d // 32, 1))).astype(np.float32)
    v = r.standard_normal((n, d)).astype(np.float32)
    nq, nk = n // bq, n // bk
    t_low = np.full((nq, nk), LOW, np.uint8)
    plan, o_ref = _fwd(q, k, v, bq, bk, t_low, 1)
    assert not np.any(plan["refine"]["qr"]) and not np.any(plan["refine"]["kr"])
    _, o_skim = _fwd(q, k, v, bq, bk, np.where(t_low == LOW, SKIM, t_low).astype(np.uint8), 0)
    assert np.max(np.abs(o_ref - o_skim)) < 1e-12


def test_refined_low_tiles_use_the_refine_operands():
    """General inputs: the refined forward differs from the E4M3 one (it does
    not read the E4M3 codes) and, with V = 1, still returns exactly 1."""
    r = np.random.default_rng(15)
    n, d, bq, bk = 192, 64, 64, 64
    q, k = (r.standard_normal((n, d)).astype(np.float32) for _ in range(2))
    v = r.standard_normal((n, d)).astype(np.float32)
    t = np.full((3, 3), LOW, np.uint8)
    _, o_ref = _fwd(q, k, v, bq, bk, t, 1)
    _, o_e4 = _fwd(q, k, v, bq, bk, t, 0)
    assert np.max(np.abs(o_ref - o_e4)) > 1e-4
    _, o_one = _fwd(q, k, np.ones_like(v), bq, bk, t, 1)
    assert np.max(np.abs(o_one - 1.0)) < 1e-12
