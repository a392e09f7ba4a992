"""GPU parity on layouts and sizes the other suites do not reach: batch > 1
with a [B, N, H, d] memory layout (head stride d, token stride H*d), sequences
shorter than one block, and top-k with 16-key blocks.  Same bars as the main
parity suite."""
import numpy as np
import pytest

from oracle import tattn as T
from synth import CONFIGS, generate

from gpu_cases import check_forward, OracleCfg, band_mask

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _bnhd(bits):
    """bf16 bit patterns [B, H, N, d] -> a [B, H, N, d] view of a contiguous
    [B, N, H, d] device tensor."""
    import torch
    out = {}
    for n in ("q", "k", "v"):
        t = torch.from_numpy(np.ascontiguousarray(bits[n].transpose(0, 2, 1, 3)).view(np.int16))
        out[n] = t.view(torch.bfloat16).cuda().permute(0, 2, 1, 3)
    return out


def _contig(bits):
    import torch
    return {n: torch.from_numpy(bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}


def _rank_ambiguous_rows(p, k):
    """Rows whose k-th and (k+1)-th largest p agree to rounding: either side
    may keep either tile."""
    if k <= 0 or k >= p.shape[1]:
        return np.zeros(p.shape[0], bool)
    s = -np.sort(-p, axis=1)
    return np.abs(s[:, k - 1] - s[:, k]) <= 1e-12 * s[:, k - 1]


def _check_plan_and_output(cfg, g, p, dev, what):
    import tile_sparse_mixed_amd as tsm
    oc = OracleCfg(cfg)
    tiers = p.tiers()
    lists, counts = p.lists()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            q, k, v = g["q"][b, h], g["k"][b, h], g["v"][b, h]
            o = T.oracle_plan(q, k, v, oc)
            band = band_mask(o["p"], oc.tau_hi, oc.tau_lo)
            if oc.top_k:
                band |= _rank_ambiguous_rows(o["p"], oc.top_k)[:, None]
            assert np.array_equal(tiers[b, h][~band], o["tiers"][~band]), (what, b, h)
            li, co = T.build_lists(tiers[b, h])
            assert np.array_equal(lists[b, h], li) and np.array_equal(counts[b, h], co), (what, b, h)
    out, _ = check_forward(tsm, p, dev, g, cfg, OracleCfg(cfg, mode=3), what=what, log=_log)
    return out


@pytest.mark.parametrize("tiles", [(128, 64), (64, 16), (64, 8)])
def test_batch_and_token_major_layout(tiles):
    import tile_sparse_mixed_amd as tsm
    import torch
    bq, bk = tiles
    cfg = CONFIGS["small"].with_(batch=2, heads=3, grid=(4, 9, 13), block_q=bq, block_k=bk)   # N = 468
    g = generate(cfg)
    dev = _bnhd(g["bits"])
    assert dev["q"].stride() == (cfg.seq_len * cfg.heads * 64, 64, cfg.heads * 64, 1)
    p = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=bq, block_k=bk, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo,
                 out_fp32=True)
    out_t = tsm.forward(p, dev["q"], dev["k"], dev["v"])
    assert out_t.stride() == dev["q"].stride()
    o32 = out_t.cpu().numpy()
    assert np.array_equal(_check_plan_and_output(cfg, g, p, dev, f"bnhd {bq}x{bk}"), o32)
    # bf16 output in the same layout: the same tiers, each value rounded once
    p16 = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=bq, block_k=bk, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo)
    assert np.array_equal(p16.tiers(), p.tiers())
    o16 = tsm.forward(p16, dev["q"], dev["k"], dev["v"])
    assert o16.dtype == torch.bfloat16 and o16.stride() == dev["q"].stride()
    o16 = o16.float().cpu().numpy()
    assert np.all(np.abs(o16 - o32) <= np.abs(o32) * 2.0 ** -8)


@pytest.mark.parametrize("n", [1, 5, 16, 64, 65, 127])
@pytest.mark.parametrize("tiles", [(128, 64), (64, 16), (64, 8)])
def test_short_sequences(n, tiles):
    """One (partial) query block; with 16-key blocks, a few key blocks."""
    import tile_sparse_mixed_amd as tsm
    bq, bk = tiles
    cfg = CONFIGS["small"].with_(heads=2, grid=(1, 1, n), block_q=bq, block_k=bk)
    g = generate(cfg)
    dev = _contig(g["bits"])
    p = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=bq, block_k=bk, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo,
                 out_fp32=True)
    _check_plan_and_output(cfg, g, p, dev, f"N={n} {bq}x{bk}")
    pf = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=bq, block_k=bk, mode="all_full", out_fp32=True)
    outf = tsm.forward(pf, dev["q"], dev["k"], dev["v"]).cpu().numpy()
    for h in range(cfg.heads):
        ref = T.naive_attention(g["q"][0, h], g["k"][0, h], g["v"][0, h])
        assert np.abs(outf[0, h] - ref).max() <= 5e-3, (n, tiles, h)


def test_top_k_with_16_key_blocks():
    import tile_sparse_mixed_amd as tsm
    cfg = CONFIGS["fine_adaptive"].with_(grid=(2, 10, 50), heads=2, mode=0, top_k=9)   # N = 1000, Nk = 63
    g = generate(cfg)
    dev = _contig(g["bits"])
    p = tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi,
                 tau_lo=cfg.tau_lo, top_k=9, out_fp32=True)
    _check_plan_and_output(cfg, g, p, dev, "top-9 64x16")
    kept_nondiag = (p.tiers()[0] != 0) & ~T.diagonal_mask(cfg.seq_len, cfg.block_q, cfg.block_k)[None]
    assert kept_nondiag.sum(axis=2).max() <= 9
