"""Pins of plan reuse across diffusion steps (APT: attention probabilities
predicted across timesteps).  Reuse keeps the previous step's tier map and
recomputes everything else from the new step's inputs; so (1) reusing a plan
on the inputs it was routed on reproduces that plan exactly, and (2) on a new
step it equals a plan of the new inputs under the old tier map, whose pooled
parts are the new inputs' own block means and codes."""
from types import SimpleNamespace

import numpy as np

from oracle import tattn as T
from synth import CONFIGS, drift_step, generate


def _cfg(c):
    return SimpleNamespace(block_q=c.block_q, block_k=c.block_k, tau_hi=c.tau_hi, tau_lo=c.tau_lo, top_k=0,
                           mode=0, keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256)


def test_reuse_on_the_same_step_is_the_plan():
    c = CONFIGS["small"].with_(heads=1)
    g = generate(c)
    q, k, v = g["q"][0, 0], g["k"][0, 0], g["v"][0, 0]
    p0 = T.oracle_plan(q, k, v, _cfg(c))
    p1 = T.oracle_replan(q, k, v, p0, _cfg(c))
    for key in ("qbar", "kbar", "vbar", "tiers", "lists", "counts", "q8", "sq", "k8", "sk", "v8", "sv"):
        assert np.array_equal(p0[key], p1[key]), key
    o0 = T.oracle_forward(q, k, v, p0, c.block_q, c.block_k)
    o1 = T.oracle_forward(q, k, v, p1, c.block_q, c.block_k)
    assert np.array_equal(o0, o1)


def test_reuse_on_the_next_step_keeps_tiers_and_repools():
    c = CONFIGS["small"].with_(heads=1)
    g0 = generate(c)
    g1 = drift_step(g0, c, 1, 0.1)
    q0, k0, v0 = g0["q"][0, 0], g0["k"][0, 0], g0["v"][0, 0]
    q1, k1, v1 = g1["q"][0, 0], g1["k"][0, 0], g1["v"][0, 0]
    p0 = T.oracle_plan(q0, k0, v0, _cfg(c))
    r1 = T.oracle_replan(q1, k1, v1, p0, _cfg(c))
    assert np.array_equal(r1["tiers"], p0["tiers"])
    assert np.array_equal(r1["kbar"], T.pool_means(k1, c.block_k))
    assert np.array_equal(r1["vbar"], T.pool_means(v1, c.block_k))
    k8, sk, _ = T.quantise_blocks(k1, c.block_k)
    assert np.array_equal(r1["k8"], k8) and np.array_equal(r1["sk"], sk)
    assert not np.array_equal(r1["kbar"], p0["kbar"])
