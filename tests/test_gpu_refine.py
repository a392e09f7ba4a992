"""GPU parity of the refined low tier (low_refine = 1; "Triage": refining a
tile with 4-bit residual correction): the pooling kernel's MXFP4 copy of K
and of its residual bit for bit against the oracle's codec, and the fused
kernel's output against the oracle under the GPU's tier map, with the
probability codes admitted as for the E4M3 low tier, for 128- and 64-row
query blocks at d = 128 and 64, key blocks of 64 down to one key, ragged lengths, the threshold and adaptive
routers, fp32 and bf16 outputs; plus the code-dumping forward equal to the
plain one bit for bit."""
import numpy as np
import pytest

from oracle import mxfp4
from oracle import tattn as T
from synth import CONFIGS

from gpu_cases import check_forward, OracleCfg, band_mask, device_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "small": CONFIGS["small"].with_(heads=2),                                    # d 64, 128x64
    "small_q64": CONFIGS["small"].with_(heads=2, block_q=64),                    # two waves
    "d128_ragged": CONFIGS["wan_like"].with_(heads=2, grid=(3, 10, 23)),         # N 690
    "d128_q64": CONFIGS["wan_like"].with_(heads=2, grid=(2, 10, 50), block_q=64),
    # gathered steps: refined 16-, 8-, 4- and one-key blocks
    "fine64x16": CONFIGS["fine_adaptive"].with_(grid=(2, 10, 50), heads=2, mode=0),
    "fine128x8_d64": CONFIGS["small"].with_(grid=(5, 9, 13), heads=2, block_k=8),
    "fine64x4": CONFIGS["fine_adaptive"].with_(grid=(3, 7, 9), heads=2, mode=0, block_k=4),
    "fine64x1": CONFIGS["fine_adaptive"].with_(grid=(2, 5, 13), heads=2, mode=0, block_k=1),
}


def _log(msg):
    print(msg, flush=True)


def _plan(tsm, dev, cfg, mode="threshold", out_fp32=True):
    return tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi,
                    tau_lo=cfg.tau_lo, top_k=cfg.top_k, mode=mode, keep_min=cfg.keep_min, keep_max=cfg.keep_max,
                    full_frac=cfg.full_frac, entropy_samples=cfg.entropy_samples, out_fp32=out_fp32, low_refine=True)


def _ocfg(cfg, mode=3):
    oc = OracleCfg(cfg, mode=mode)
    oc.low_refine = 1
    return oc


@pytest.mark.parametrize("name", list(CASES))
def test_mx4_and_residual_copies_bit_exact(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    m, r = p.mx4(), p.mx4_residual()
    for h in range(cfg.heads):
        R = T.refine_operands(g["q"][0, h], g["k"][0, h])
        assert np.array_equal(m["k4"][0, h], mxfp4.pack_nibbles(R["k_codes"])), (name, h)
        assert np.array_equal(m["k4s"][0, h], R["k_scales"]), (name, h)
        assert np.array_equal(r["k4r"][0, h], mxfp4.pack_nibbles(R["kr_codes"])), (name, h)
        assert np.array_equal(r["k4rs"][0, h], R["kr_scales"]), (name, h)
    _log(f"[refine {name}] K codes, residual codes and scales bit-exact")


@pytest.mark.parametrize("mode", ["threshold", "adaptive"])
@pytest.mark.parametrize("name", list(CASES))
def test_refined_forward_parity(name, mode):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    if mode == "adaptive":
        cfg = cfg.with_(mode=1)
    g, dev = device_inputs(cfg)
    for out_fp32 in (True, False):
        p = _plan(tsm, dev, cfg, mode=mode, out_fp32=out_fp32)
        tiers = p.tiers()
        assert np.any(tiers == T.LOW), name
        out, _ = check_forward(tsm, p, dev, g, cfg, _ocfg(cfg), what=f"refine {name} {mode} {'fp32' if out_fp32 else 'bf16'}",
                               log=_log)
        plain = tsm.forward(p, dev["q"], dev["k"], dev["v"]).float().cpu().numpy()
        assert np.array_equal(plain, out), (name, mode, out_fp32)
        if out_fp32 and mode == "threshold":
            # tiers under low_refine are the router's, as without it
            oc = OracleCfg(cfg)
            for h in range(cfg.heads):
                o = T.oracle_plan(g["q"][0, h], g["k"][0, h], g["v"][0, h], oc)
                band = band_mask(o["p"], oc.tau_hi, oc.tau_lo)
                assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), (name, h)
