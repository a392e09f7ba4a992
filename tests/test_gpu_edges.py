"""GPU parity at the edges the ABI allows: the largest key-block count the
router and the fused kernel hold (4096 key blocks, with 64- and 16-key
blocks), all-zero blocks (amax 0, scale 1), top-k at its extremes and equal
thresholds (no low tier).  Same bars as the main parity suite; at the largest
sizes the output is checked on sampled query blocks."""
import numpy as np
import pytest

from oracle import tattn as T
from synth import CONFIGS, generate
from synth.gen import to_bf16_bits, bf16_bits_to_f32

from gpu_cases import check_forward, OracleCfg, band_mask

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _dev(bits):
    import torch
    return {n: torch.from_numpy(bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}


def _plan(tsm, cfg, d, **kw):
    args = dict(block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo,
                top_k=cfg.top_k, out_fp32=True)
    args.update(kw)
    return tsm.plan(d["q"], d["k"], d["v"], **args)


def _check(cfg, g, p, d, rows=None, top_k=None, what=""):
    import tile_sparse_mixed_amd as tsm
    oc = OracleCfg(cfg, top_k=top_k)
    tiers = p.tiers()
    for h in range(cfg.heads):
        q, k, v = g["q"][0, h], g["k"][0, h], g["v"][0, h]
        o = T.oracle_plan(q, k, v, oc)
        band = band_mask(o["p"], oc.tau_hi, oc.tau_lo)
        if oc.top_k and 0 < oc.top_k < o["p"].shape[1]:
            srt = -np.sort(-o["p"], axis=1)
            band |= (np.abs(srt[:, oc.top_k - 1] - srt[:, oc.top_k]) <= 1e-12 * srt[:, oc.top_k - 1])[:, None]
        assert np.array_equal(tiers[0, h][~band], o["tiers"][~band]), (what, h)
        _log(f"  {what} h{h}: tiers F/L/S {[round(float((tiers[0, h] == x).mean()), 4) for x in (2, 1, 0)]}")
    check_forward(tsm, p, d, g, cfg, OracleCfg(cfg, mode=3), rows=rows, what=what, log=_log)


@pytest.mark.parametrize("bk", [64, 16, 1])
def test_largest_key_block_count(bk):
    """4096 key blocks: N = 262144 tokens at 64-key blocks (d = 64, 128-row
    query blocks), N = 65536 at 16-key blocks (d = 128, 64-row query blocks),
    N = 4096 at one-key blocks (d = 128, 64-row query blocks)."""
    import tile_sparse_mixed_amd as tsm
    if bk == 64:
        cfg = CONFIGS["small"].with_(heads=1, grid=(64, 64, 64))
    elif bk == 16:
        cfg = CONFIGS["fine_adaptive"].with_(heads=1, grid=(16, 64, 64), mode=0)
    else:
        cfg = CONFIGS["fine_adaptive"].with_(heads=1, grid=(4, 32, 32), mode=0, block_k=1)
    assert cfg.n_kblocks == 4096
    _log(f"[max Nk] N={cfg.seq_len} d={cfg.head_dim} tiles {cfg.block_q}x{cfg.block_k}")
    g = generate(cfg)
    d = _dev(g["bits"])
    p = _plan(tsm, cfg, d)
    nq = cfg.n_qblocks
    _check(cfg, g, p, d, rows=[0, nq // 3, nq - 1], what=f"maxNk bk{bk}")


def _zeroed(cfg):
    g = generate(cfg)
    bits = {n: g["bits"][n].copy() for n in ("q", "k", "v")}
    bq, bk = cfg.block_q, cfg.block_k
    bits["k"][:, :, 3 * bk:4 * bk] = 0          # an all-zero key block
    bits["v"][:, :, 5 * bk:6 * bk] = 0          # an all-zero value block
    bits["q"][:, :, 1 * bq:2 * bq] = 0          # an all-zero query block
    bits["v"][:, :, -7:] = 0                    # zeros inside the ragged last block
    for n in ("q", "k", "v"):
        g[n] = bf16_bits_to_f32(bits[n])
    g["bits"] = bits
    return g


def test_all_zero_blocks():
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["wan_like"].with_(heads=2, grid=(3, 10, 23))        # N = 690
    g = _zeroed(cfg)
    d = _dev(g["bits"])
    p = _plan(tsm, cfg, d)
    pool = p.pool()
    assert np.all(pool["sk"][0, :, 3] == 1.0) and np.all(pool["sv"][0, :, 5] == 1.0)
    assert np.all(pool["sq"][0, :, 1] == 1.0)
    _check(cfg, g, p, d, what="zero blocks")


@pytest.mark.parametrize("top_k", [1, 32])
def test_top_k_extremes(top_k):
    """top_k = 1 keeps one tile per row besides the diagonal; top_k = Nk keeps all."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["small"].with_(heads=2, top_k=top_k)                  # Nk = 32
    g = generate(cfg)
    d = _dev(g["bits"])
    p = _plan(tsm, cfg, d)
    _check(cfg, g, p, d, top_k=top_k, what=f"top_k {top_k}")
    if top_k == 1:
        diag = T.diagonal_mask(cfg.seq_len, cfg.block_q, cfg.block_k)
        assert np.all(((p.tiers()[0] != 0) & ~diag).sum(axis=2) <= 1)


def test_equal_thresholds_have_no_low_tier():
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["small"].with_(heads=2, tau_hi=0.004, tau_lo=0.004)
    g = generate(cfg)
    d = _dev(g["bits"])
    p = _plan(tsm, cfg, d)
    assert not np.any(p.tiers() == 1)
    _check(cfg, g, p, d, what="tau_hi == tau_lo")


@pytest.mark.parametrize("bk", [16, 8, 4, 1])
def test_adaptive_rows_at_the_list_bound(bk):
    """keep_min = keep_max = 0.5 makes every head's k_h = ceil(0.5 Nk): each
    row keeps k_h tiles plus any diagonal block outside them, the most the
    fused kernel's list (sized by that bound) has to hold."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["fine_adaptive"].with_(heads=2, grid=(2, 10, 50), block_k=bk, keep_min=0.5, keep_max=0.5)
    g = generate(cfg)
    d = _dev(g["bits"])
    p = tsm.plan(d["q"], d["k"], d["v"], block_q=cfg.block_q, block_k=bk, mode="adaptive", keep_min=0.5,
                 keep_max=0.5, full_frac=cfg.full_frac, entropy_samples=cfg.entropy_samples, out_fp32=True)
    kh = p.kh()[0]
    assert np.all(kh == int(np.ceil(0.5 * cfg.n_kblocks)))
    tiers = p.tiers()
    kept = (tiers != 0).sum(axis=3)
    _log(f"[list bound bk{bk}] k_h {kh.tolist()}, kept per row {int(kept.min())}..{int(kept.max())} of {cfg.n_kblocks}")
    check_forward(tsm, p, d, g, cfg, OracleCfg(cfg, mode=3), what=f"list bound bk{bk}", log=_log)


def test_top_k_rows_at_the_list_bound():
    """top_k with every tile above the thresholds: rows keep exactly top_k
    tiles plus the diagonal blocks, the list bound for top-k plans."""
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["small"].with_(heads=2, tau_hi=0.0, tau_lo=0.0, top_k=5)
    g = generate(cfg)
    d = _dev(g["bits"])
    p = _plan(tsm, cfg, d)
    kept = (p.tiers() != 0).sum(axis=3)
    assert kept.min() >= 5
    _check(cfg, g, p, d, top_k=5, what="top_k at bound")
