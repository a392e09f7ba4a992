"""GPU parity of plan reuse across diffusion steps (tattn_replan): after a drift
step the plan keeps its tiers and lists, its pooled statistics are the new
inputs' own, and the output matches the oracle's reuse of the old tier map on
the new inputs.  Reusing on unchanged inputs reproduces the forward bit for
bit; a forward with the previous step's K is refused."""
import numpy as np
import pytest

from oracle import tattn as T
from synth import CONFIGS, drift_step, generate

from gpu_cases import check_forward, OracleCfg

pytestmark = pytest.mark.gpu

CASES = {
    "small": CONFIGS["small"].with_(heads=2),
    "d128_ragged": CONFIGS["wan_like"].with_(heads=2, grid=(3, 10, 23)),
    "fine64x16": CONFIGS["fine_adaptive"].with_(heads=2, grid=(2, 10, 50)),
}


def _log(msg):
    print(msg, flush=True)


def _dev(g):
    import torch
    return {n: torch.from_numpy(g["bits"][n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}


def _plan(tsm, cfg, d, mode):
    return tsm.plan(d["q"], d["k"], d["v"], block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi,
                    tau_lo=cfg.tau_lo, mode=mode, keep_min=cfg.keep_min, keep_max=cfg.keep_max,
                    full_frac=cfg.full_frac, entropy_samples=cfg.entropy_samples, out_fp32=True)


@pytest.mark.parametrize("name", list(CASES))
def test_replan_after_a_drift_step(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    mode = "adaptive" if cfg.mode == 1 else "threshold"
    g0 = generate(cfg)
    g1 = drift_step(g0, cfg, 1, 0.1)
    d0, d1 = _dev(g0), _dev(g1)
    p = _plan(tsm, cfg, d0, mode)
    t0 = p.tiers()
    l0, c0 = p.lists()
    tsm.replan(p, d1["q"], d1["k"], d1["v"])
    assert np.array_equal(p.tiers(), t0)
    l1, c1 = p.lists()
    assert np.array_equal(l1, l0) and np.array_equal(c1, c0)
    pool = p.pool()
    fresh = _plan(tsm, cfg, d1, mode).tiers()
    _log(f"[replan {name}] tiles whose tier a fresh routing would change: {np.mean(fresh != t0):.4f}")
    oc = OracleCfg(cfg)
    for h in range(cfg.heads):
        q1, k1, v1 = g1["q"][0, h], g1["k"][0, h], g1["v"][0, h]
        prev = {"tiers": t0[0, h]}
        r = T.oracle_replan(q1, k1, v1, prev, oc)
        assert np.array_equal(pool["qbar"][0, h], r["qbar"]) and np.array_equal(pool["kbar"][0, h], r["kbar"])
        assert np.array_equal(pool["vbar"][0, h], r["vbar"]) and np.array_equal(pool["sk"][0, h], r["sk"])
    # the oracle's plan reuse is its plan under the previous step's tier map
    check_forward(tsm, p, d1, g1, cfg, OracleCfg(cfg, mode=3), what=f"replan {name}", log=_log)


def test_replan_on_the_same_inputs_is_bit_identical_and_rebinds_k_v():
    import torch
    import tile_sparse_mixed_amd as tsm
    cfg = CASES["small"]
    g0 = generate(cfg)
    d0 = _dev(g0)
    p = _plan(tsm, cfg, d0, "threshold")
    a = tsm.forward(p, d0["q"], d0["k"], d0["v"]).clone()
    d0b = {n: t.clone() for n, t in d0.items()}
    tsm.replan(p, d0b["q"], d0b["k"], d0b["v"])
    b = tsm.forward(p, d0b["q"], d0b["k"], d0b["v"])
    assert torch.equal(a, b)
    with pytest.raises(tsm.TattnError):
        tsm.forward(p, d0["q"], d0["k"], d0["v"])     # the plan now belongs to the new K and V


@pytest.mark.parametrize("name", ["small", "d128_ragged"])
def test_forward_with_new_q_takes_its_own_q_scales(name):
    """A forward given queries other than the ones the plan was routed with
    (same K and V, no replan): the tiers stay the plan's, and the LOW tier's
    per-block E4M3 Q scales come from the new queries.  The new queries are
    the next step's, times 4 (exact in bf16), so every block's amax differs
    from the routed one: with the routed scales the E4M3 copy of Q would
    saturate.  Compared with the oracle under the plan's tiers on the new
    queries."""
    import tile_sparse_mixed_amd as tsm
    from synth.gen import bf16_bits_to_f32, to_bf16_bits
    cfg = CASES[name]
    g0 = generate(cfg)
    q_new = 4.0 * drift_step(g0, cfg, 1, 0.1)["q"]
    g = dict(g0)
    g["bits"] = dict(g0["bits"])
    g["bits"]["q"] = to_bf16_bits(q_new)
    g["q"] = bf16_bits_to_f32(g["bits"]["q"]).astype(np.float32)
    assert np.array_equal(g["q"], q_new)
    d0 = _dev(g0)
    d = dict(d0, q=_dev(g)["q"])      # the plan's own K and V tensors
    p = _plan(tsm, cfg, d0, "threshold")
    t0 = p.tiers()
    assert (t0 == 1).any(), "the case must have LOW tiles"
    check_forward(tsm, p, d, g, cfg, OracleCfg(cfg, mode=3), what=f"new q {name}", log=_log)
    assert np.array_equal(p.tiers(), t0)
