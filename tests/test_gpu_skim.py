"""GPU parity of the MXFP4 SKIM tier (tau_skim > 0): the pooling kernel's
MXFP4 copies of K and V bit for bit against the oracle's codec, the four-tier
threshold map and its lists against the oracle outside the threshold bands,
the fused kernel's output under the GPU's tiers and under random external
four-tier maps, the full-size Wan-like shape and the largest key-block count
on sampled query blocks, all-zero blocks, top-k, and plan reuse."""
import numpy as np
import pytest

from oracle import mxfp4
from oracle import tattn as T
from synth import CONFIGS

from gpu_cases import OracleCfg, band_mask, device_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "small": CONFIGS["small"].with_(heads=2, tau_skim=3e-4),                                   # d 64, 128x64
    "small_q64": CONFIGS["small"].with_(heads=2, block_q=64, tau_skim=3e-4),                   # two waves
    "d128_ragged": CONFIGS["wan_like"].with_(heads=2, grid=(3, 10, 23), tau_skim=1e-4),        # N 690
    "d128_q64": CONFIGS["wan_like"].with_(heads=2, grid=(2, 10, 50), block_q=64, tau_skim=1e-4),
}


def _log(msg):
    print(msg, flush=True)


def _plan(tsm, dev, cfg, mode="threshold", out_fp32=True):
    return tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi,
                    tau_lo=cfg.tau_lo, top_k=cfg.top_k, mode=mode, out_fp32=out_fp32, tau_skim=cfg.tau_skim)


def _check_out(out, ref, what, rows=None, bq=None):
    if rows is not None:
        sel = np.concatenate([np.arange(I * bq, min(out.shape[0], (I + 1) * bq)) for I in rows])
        out, ref = out[sel], ref[sel]
    err = np.abs(out.astype(np.float64) - ref)
    _log(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (what, err.max(), err.mean())


@pytest.mark.parametrize("name", list(CASES))
def test_mx4_copies_bit_exact(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    m = p.mx4()
    for h in range(cfg.heads):
        kc, ks, _ = mxfp4.quantise(g["k"][0, h])
        _, _, vd = mxfp4.quantise(g["v"][0, h])
        assert np.array_equal(m["k4"][0, h], mxfp4.pack_nibbles(kc)), (name, h)
        assert np.array_equal(m["k4s"][0, h], ks), (name, h)
        assert np.array_equal(m["vskim"][0, h].view(np.uint16), vd.astype(np.float16).view(np.uint16)), (name, h)
    _log(f"[mx4 {name}] codes, scales and values bit-exact")


@pytest.mark.parametrize("name", list(CASES))
def test_four_tier_threshold_parity(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    tiers = p.tiers()
    lists, counts = p.lists()
    st = p.stats()
    assert st["n_skim"] == int((tiers == T.SKIM).sum()) > 0
    _log(f"[skim {name}] FULL/LOW/SKIM/SKIP {[round(float((tiers == x).mean()), 3) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    for h in range(cfg.heads):
        q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
        o = T.oracle_plan(q, k, v, oc)
        band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
        assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), (name, h)
        li, co = T.build_lists(tiers[0, h])
        assert np.array_equal(lists[0, h], li) and np.array_equal(counts[0, h], co), (name, h)
        oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=tiers[0, h])
        _check_out(out[0, h], T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k), f"h{h}")


@pytest.mark.parametrize("name,seed", [("small", 1), ("d128_ragged", 2), ("d128_q64", 3)])
def test_external_four_tier_maps(name, seed):
    """Random maps over all four tiers, and a map that is SKIM everywhere but
    the diagonal."""
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    nq, nk = cfg.n_qblocks, cfg.n_kblocks
    r = np.random.default_rng(seed)
    oc = OracleCfg(cfg, mode=3)
    for what, t in (("random", r.integers(0, 4, (1, cfg.heads, nq, nk))),
                    ("all_skim", np.full((1, cfg.heads, nq, nk), T.SKIM))):
        p = _plan(tsm, dev, cfg, mode="external")
        p.set_tiers(t.astype(np.uint8))
        out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
        tg = p.tiers()
        for h in range(cfg.heads):
            q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
            oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=t[0, h])
            assert np.array_equal(tg[0, h], oe["tiers"])
            _check_out(out[0, h], T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k), f"{name} {what} h{h}")


def test_skim_bytes_need_the_tier():
    """Without tau_skim a SKIM byte is refused and the plan is left unchanged."""
    import tile_sparse_mixed_amd as tsm
    cfg = CASES["small"].with_(tau_skim=0.0)
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg, mode="external")
    with pytest.raises(tsm.TattnError):
        p.set_tiers(np.full((1, cfg.heads, cfg.n_qblocks, cfg.n_kblocks), T.SKIM, np.uint8))
    with pytest.raises(tsm.TattnError):
        p.mx4()


def test_full_size_wan_shape_sampled():
    """32760 tokens x d 128 at 128x64 tiles with the SKIM tier (two of the
    workload's heads): tiers and lists exact outside the bands, output on three
    query blocks including the ragged last one."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["wan_skim"]
    g, dev = device_inputs(cfg, heads=[0, 7])
    p = _plan(tsm, dev, cfg)
    out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    tiers = p.tiers()
    lists, counts = p.lists()
    _log(f"[skim full size] FULL/LOW/SKIM/SKIP {[round(float((tiers == x).mean()), 4) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    rows = [0, cfg.n_qblocks // 2, cfg.n_qblocks - 1]
    for h in range(2):
        q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
        o = T.oracle_plan(q, k, v, oc)
        band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
        assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), h
        li, co = T.build_lists(tiers[0, h])
        assert np.array_equal(lists[0, h], li) and np.array_equal(counts[0, h], co), h
        oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=tiers[0, h])
        ref = T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k, rows=rows)
        _check_out(out[0, h], ref, f"full size h{h}", rows=rows, bq=cfg.block_q)


def test_zero_blocks_in_skim_tiles():
    """All-zero K, V and Q blocks and zeros inside the ragged last block, every
    non-diagonal tile SKIM: scale byte 0 (2^-127) for the zero rows and an
    exact zero contribution from their codes."""
    import tile_sparse_mixed_amd as tsm
    from synth.gen import bf16_bits_to_f32
    cfg = CASES["d128_ragged"]
    g, _ = device_inputs(cfg)
    import torch
    bits = {n: g["bits"][n].copy() for n in ("q", "k", "v")}
    bits["k"][:, :, 3 * 64:4 * 64] = 0
    bits["v"][:, :, 5 * 64:6 * 64] = 0
    bits["q"][:, :, 128:256] = 0
    bits["v"][:, :, -7:] = 0
    for n in ("q", "k", "v"):
        g[n] = bf16_bits_to_f32(bits[n])
    dev = {n: torch.from_numpy(bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    p = _plan(tsm, dev, cfg, mode="external")
    t = np.full((1, cfg.heads, cfg.n_qblocks, cfg.n_kblocks), T.SKIM, np.uint8)
    p.set_tiers(t)
    out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    m = p.mx4()
    assert np.all(m["k4s"][0, :, 3 * 64:4 * 64] == 0) and np.all(m["k4"][0, :, 3 * 64:4 * 64] == 0)
    oc = OracleCfg(cfg, mode=3)
    for h in range(cfg.heads):
        q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
        oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=t[0, h])
        _check_out(out[0, h], T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k), f"zero blocks h{h}")


def test_replan_keeps_skim_tiles_and_refreshes_mx4():
    from synth import drift_step
    import tile_sparse_mixed_amd as tsm
    import torch
    cfg = CASES["d128_ragged"]
    g0, dev0 = device_inputs(cfg)
    g1 = drift_step(g0, cfg, 1, 0.1)
    dev1 = {n: torch.from_numpy(g1["bits"][n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    p = _plan(tsm, dev0, cfg)
    t0 = p.tiers()
    assert np.any(t0 == T.SKIM)
    tsm.replan(p, dev1["q"], dev1["k"], dev1["v"])
    out = tsm.forward(p, dev1["q"], dev1["k"], dev1["v"]).cpu().numpy()
    assert np.array_equal(p.tiers(), t0)
    m = p.mx4()
    oc = OracleCfg(cfg)
    for h in range(cfg.heads):
        q1, k1, v1 = g1["q"][0, h], g1["k"][0, h], g1["v"][0, h]
        kc, ks, _ = mxfp4.quantise(k1)
        assert np.array_equal(m["k4"][0, h], mxfp4.pack_nibbles(kc)) and np.array_equal(m["k4s"][0, h], ks)
        r = T.oracle_replan(q1, k1, v1, {"tiers": t0[0, h]}, oc)
        _check_out(out[0, h], T.oracle_forward(q1, k1, v1, r, cfg.block_q, cfg.block_k), f"replan h{h}")


def test_top_k_with_four_tiers():
    import tile_sparse_mixed_amd as tsm
    cfg = CASES["small"].with_(top_k=12)
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    tiers = p.tiers()
    oc = OracleCfg(cfg)
    for h in range(cfg.heads):
        q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
        o = T.oracle_plan(q, k, v, oc)
        band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
        srt = -np.sort(-o["p"], axis=1)
        band |= (np.abs(srt[:, 11] - srt[:, 12]) <= 1e-12 * srt[:, 11])[:, None]
        assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), h
        diag = T.diagonal_mask(cfg.seq_len, cfg.block_q, cfg.block_k)
        assert np.all(((tiers[0, h] != T.SKIP) & ~diag).sum(axis=1) <= 12)
        oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=tiers[0, h])
        _check_out(out[0, h], T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k), f"top-k h{h}")


def test_largest_key_block_count_with_skim():
    """4096 key blocks (N = 262144, d = 64, 128x64 tiles) with the SKIM tier:
    tiers and lists outside the bands, output on three sampled query blocks."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["small"].with_(heads=1, grid=(64, 64, 64), tau_skim=1e-4)
    assert cfg.n_kblocks == 4096
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    out = tsm.forward(p, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    tiers = p.tiers()
    _log(f"[skim max Nk] FULL/LOW/SKIM/SKIP {[round(float((tiers == x).mean()), 4) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    q, k, v = g["q"][0, 0], g["k"][0, 0], g["v"][0, 0]
    o = T.oracle_plan(q, k, v, oc)
    band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
    assert np.array_equal(tiers[0, 0][~band], o["tiers"][~band])
    rows = [0, cfg.n_qblocks // 3, cfg.n_qblocks - 1]
    oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=tiers[0, 0])
    ref = T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k, rows=rows)
    _check_out(out[0, 0], ref, "max Nk", rows=rows, bq=cfg.block_q)
