"""GPU parity of the MXFP4 SKIM tier (tau_skim > 0): the pooling kernel's
MXFP4 copy of K bit for bit against the oracle's codec, the four-tier
threshold map and its lists against the oracle outside the threshold bands,
the fused kernel's output under the GPU's tiers and under random external
four-tier maps, the full-size Wan-like shape and the largest key-block count
on sampled query blocks, all-zero blocks, top-k, and plan reuse."""
import numpy as np
import pytest

from oracle import mxfp4
from oracle import tattn as T
from synth import CONFIGS, generate

from gpu_cases import check_forward, OracleCfg, band_mask, device_inputs, device_tiled, sample_rows, TiledHeads

pytestmark = pytest.mark.gpu

CASES = {
    "small": CONFIGS["small"].with_(heads=2, tau_skim=3e-4),                                   # d 64, 128x64
    "small_q64": CONFIGS["small"].with_(heads=2, block_q=64, tau_skim=3e-4),                   # two waves
    "d128_ragged": CONFIGS["wan_like"].with_(heads=2, grid=(3, 10, 23), tau_skim=1e-4),        # N 690
    "d128_q64": CONFIGS["wan_like"].with_(heads=2, grid=(2, 10, 50), block_q=64, tau_skim=1e-4),
    # gathered steps: four 16-key or eight 8-key SKIM blocks per step
    "fine64x16": CONFIGS["fine_adaptive"].with_(grid=(2, 10, 50), heads=2, mode=0, tau_skim=1e-4),   # N 1000, Nk 63
    "fine64x8": CONFIGS["fine_adaptive"].with_(grid=(3, 7, 9), heads=2, mode=0, block_k=8, tau_skim=1e-4),
    "fine64x8_d64": CONFIGS["small"].with_(heads=2, grid=(5, 9, 13), block_q=64, block_k=8, tau_skim=3e-4),
    "fine128x16_d64": CONFIGS["small"].with_(heads=2, grid=(5, 9, 13), block_k=16, tau_skim=3e-4),
    # blocks below 8 keys: 16, 32 or 64 SKIM blocks per step
    "fine64x4": CONFIGS["fine_adaptive"].with_(grid=(3, 7, 9), heads=2, mode=0, block_k=4, tau_skim=1e-4),
    "fine128x2_d64": CONFIGS["small"].with_(heads=2, grid=(3, 7, 9), block_k=2, tau_skim=3e-4),
    "fine64x1": CONFIGS["fine_adaptive"].with_(grid=(2, 5, 13), heads=2, mode=0, block_k=1, tau_skim=1e-4),
}


def _log(msg):
    print(msg, flush=True)


def _plan(tsm, dev, cfg, mode="threshold", out_fp32=True):
    return tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi,
                    tau_lo=cfg.tau_lo, top_k=cfg.top_k, mode=mode, out_fp32=out_fp32, tau_skim=cfg.tau_skim)


@pytest.mark.parametrize("name", list(CASES))
def test_mx4_copies_bit_exact(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    m = p.mx4()
    for h in range(cfg.heads):
        kc, ks, _ = mxfp4.quantise(g["k"][0, h])
        assert np.array_equal(m["k4"][0, h], mxfp4.pack_nibbles(kc)), (name, h)
        assert np.array_equal(m["k4s"][0, h], ks), (name, h)
    _log(f"[mx4 {name}] codes and scales bit-exact")


@pytest.mark.parametrize("name", list(CASES))
def test_four_tier_threshold_parity(name):
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name]
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
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
    check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), what=f"skim {name}", log=_log)


@pytest.mark.parametrize("name,seed", [("small", 1), ("d128_ragged", 2), ("d128_q64", 3), ("fine64x16", 4),
                                       ("fine64x8_d64", 5), ("fine128x16_d64", 6), ("fine64x4", 7),
                                       ("fine128x2_d64", 8), ("fine64x1", 9)])
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
        tg = p.tiers()
        for h in range(cfg.heads):
            q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
            oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=t[0, h])
            assert np.array_equal(tg[0, h], oe["tiers"])
        check_forward(tsm, p, dev, g, cfg, oc, what=f"{name} {what}", log=_log)


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


@pytest.mark.parametrize("wl", ["wan_skim", "fine_skim"])
def test_full_size_wan_shape_sampled(wl):
    """The SKIM tier in the full launch: 32760 tokens x 40 heads x d 128 at
    128x64 (and 64x16) tiles, four distinct generated heads tiled to 40.
    Tiers and lists exact outside the bands on the sampled heads, and 32
    query blocks per sampled head (the first, the ragged last, the most-LOW
    and most-FULL rows, evenly spaced ones) against the oracle under the GPU's
    tiers; the plain forward equal to the code-dumping one bit for bit."""
    import torch
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS[wl]
    gen_heads, sample_heads = 4, [0, 13, 26, 39]
    g = generate(cfg.with_(heads=gen_heads))
    dev = device_tiled(g["bits"], cfg.heads)
    p = _plan(tsm, dev, cfg, out_fp32=False)
    plain = tsm.forward(p, dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    tiers = p.tiers()
    lists, counts = p.lists()
    _log(f"[skim full size {wl}] FULL/LOW/SKIM/SKIP {[round(float((tiers == x).mean()), 4) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    for h in sample_heads:
        src = h % gen_heads
        o = T.oracle_plan(g["q"][0, src], g["k"][0, src], g["v"][0, src], oc)
        band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
        assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), h
        li, co = T.build_lists(tiers[0, h])
        assert np.array_equal(lists[0, h], li) and np.array_equal(counts[0, h], co), h
    nq = cfg.n_qblocks
    out, _ = check_forward(tsm, p, dev, TiledHeads(g, gen_heads), cfg, OracleCfg(cfg, mode=3),
                           rows=lambda b, h, t: sample_rows(nq, 32, t), heads=[(0, h) for h in sample_heads],
                           what=f"skim full size {wl}", log=_log)
    assert np.array_equal(plain.float().cpu().numpy(), out), wl


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
    m = p.mx4()
    assert np.all(m["k4s"][0, :, 3 * 64:4 * 64] == 0) and np.all(m["k4"][0, :, 3 * 64:4 * 64] == 0)
    check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), what="zero blocks", log=_log)


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
    assert np.array_equal(p.tiers(), t0)
    m = p.mx4()
    for h in range(cfg.heads):
        kc, ks, _ = mxfp4.quantise(g1["k"][0, h])
        assert np.array_equal(m["k4"][0, h], mxfp4.pack_nibbles(kc)) and np.array_equal(m["k4s"][0, h], ks)
    check_forward(tsm, p, dev1, g1, cfg, OracleCfg(cfg, mode=3), what="skim replan", log=_log)


def test_top_k_with_four_tiers():
    import tile_sparse_mixed_amd as tsm
    cfg = CASES["small"].with_(top_k=12)
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
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
    check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), what="skim top-k", log=_log)


def test_largest_key_block_count_with_skim():
    """4096 key blocks (N = 262144, d = 64, 128x64 tiles) with the SKIM tier:
    tiers and lists outside the bands, output on three sampled query blocks."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["small"].with_(heads=1, grid=(64, 64, 64), tau_skim=1e-4)
    assert cfg.n_kblocks == 4096
    g, dev = device_inputs(cfg)
    p = _plan(tsm, dev, cfg)
    tiers = p.tiers()
    _log(f"[skim max Nk] FULL/LOW/SKIM/SKIP {[round(float((tiers == x).mean()), 4) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    q, k, v = g["q"][0, 0], g["k"][0, 0], g["v"][0, 0]
    o = T.oracle_plan(q, k, v, oc)
    band = band_mask(o["p"], oc.tau_hi, oc.tau_lo, tau_skim=oc.tau_skim)
    assert np.array_equal(tiers[0, 0][~band], o["tiers"][~band])
    rows = [0, cfg.n_qblocks // 3, cfg.n_qblocks - 1]
    check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), rows=rows, what="skim max Nk", log=_log)


def _rank_ambiguous_rows(p, k):
    """Rows whose k-th and (k+1)-th largest p are equal to rounding (either
    side may keep either tile)."""
    if k <= 0 or k >= p.shape[1]:
        return np.zeros(p.shape[0], bool)
    s = -np.sort(-p, axis=1)
    return np.abs(s[:, k - 1] - s[:, k]) <= 1e-12 * s[:, k - 1]


@pytest.mark.parametrize("name", ["small", "fine64x16", "fine64x4", "fine64x1"])
def test_adaptive_mode_with_skim(name):
    """Head-adaptive tiers with the fourth tier: the top k_h tiles as without
    it, the rest SKIM where p >= tau_skim and SKIP below; lists and the output
    under the GPU's map."""
    import tile_sparse_mixed_amd as tsm
    cfg = CASES[name].with_(mode=1)
    g, dev = device_inputs(cfg)
    p = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k, mode="adaptive",
                 keep_min=cfg.keep_min, keep_max=cfg.keep_max, full_frac=cfg.full_frac,
                 entropy_samples=cfg.entropy_samples, tau_skim=cfg.tau_skim, out_fp32=True)
    kh, _ = p.kh()
    tiers = p.tiers()
    lists, counts = p.lists()
    assert p.stats()["n_skim"] == int((tiers == T.SKIM).sum()) > 0
    _log(f"[adaptive skim {name}] k_h {kh.tolist()} FULL/LOW/SKIM/SKIP "
         f"{[round(float((tiers == x).mean()), 3) for x in (2, 1, 3, 0)]}")
    oc = OracleCfg(cfg)
    for h in range(cfg.heads):
        o = T.oracle_plan(g["q"][0, h], g["k"][0, h], g["v"][0, h], oc)
        if kh[h] != o["k_h"]:
            continue        # k_h on an integer boundary of r_h * Nk (checked in the three-tier tests)
        nfull = int(np.ceil(oc.full_frac * o["k_h"]))
        amb = _rank_ambiguous_rows(o["p"], o["k_h"]) | _rank_ambiguous_rows(o["p"], nfull)
        band = np.abs(o["p"] - oc.tau_skim) <= 1e-5 * oc.tau_skim
        ok = ~amb[:, None] & ~band
        assert np.array_equal(tiers[0, h][ok], o["tiers"][ok]), (name, h)
        li, co = T.build_lists(tiers[0, h])
        assert np.array_equal(lists[0, h], li) and np.array_equal(counts[0, h], co), (name, h)
    check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), what=f"adaptive skim {name}", log=_log)
