"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
oracle per head, and comparisons.  Not a test module."""
import numpy as np

from oracle import tattn as T
from synth import generate
from synth.gen import to_bf16_bits, bf16_bits_to_f32


def as_f32(x):
    """Round to a float32 representable value (the ABI takes float32 parameters)."""
    return float(np.float32(x))


def device_inputs(cfg, heads=None, seed=0):
    """Generate the workload, round fp32 inputs to bf16 once (the GPU path is
    bf16; the oracle consumes the same rounded values) and move them to cuda:0."""
    import torch
    g = generate(cfg, seed=seed, heads=heads)
    bits = g["bits"]
    if bits is None:
        bits = {n: to_bf16_bits(g[n]) for n in ("q", "k", "v")}
        for n in ("q", "k", "v"):
            g[n] = bf16_bits_to_f32(bits[n])
    dev = {n: torch.from_numpy(bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    return g, dev


class OracleCfg:
    def __init__(self, cfg, mode=None, top_k=None):
        self.block_q, self.block_k = cfg.block_q, cfg.block_k
        self.tau_hi, self.tau_lo = as_f32(cfg.tau_hi), as_f32(cfg.tau_lo)
        self.top_k = cfg.top_k if top_k is None else top_k
        self.mode = cfg.mode if mode is None else mode
        self.keep_min, self.keep_max = as_f32(cfg.keep_min), as_f32(cfg.keep_max)
        self.full_frac = as_f32(cfg.full_frac)
        self.entropy_samples = cfg.entropy_samples
        self.tau_skim = as_f32(cfg.tau_skim)
        self.low_refine = 0      # set to 1 for the refined low tier


def oracle_head(g, b, h, ocfg, mode=None, external=None):
    q, k, v = g["q"][b, h], g["k"][b, h], g["v"][b, h]
    return T.oracle_plan(q, k, v, ocfg, mode=mode, external_tiers=external)


def band_mask(p, tau_hi, tau_lo, rel=1e-5, tau_skim=0.0):
    m = (np.abs(p - tau_hi) <= rel * tau_hi) | (np.abs(p - tau_lo) <= rel * tau_lo)
    if tau_skim > 0:
        m |= np.abs(p - tau_skim) <= rel * tau_skim
    return m


def gpu_plan(dev, cfg, mode=None, out_fp32=True, top_k=None):
    import tile_sparse_mixed_amd as tsm
    m = cfg.mode if mode is None else mode
    return tsm.plan(dev["q"], dev["k"], dev["v"], block_q=cfg.block_q, block_k=cfg.block_k,
                    tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo, top_k=cfg.top_k if top_k is None else top_k,
                    mode=m, keep_min=cfg.keep_min, keep_max=cfg.keep_max, full_frac=cfg.full_frac,
                    entropy_samples=cfg.entropy_samples, out_fp32=out_fp32)


# ---------------------------------------------------------------------------
# Probability codes of quantised (LOW, SKIM) tiles.  Where the oracle's
# x = fl32(448 e^{s - m_t}) lies on a rounding midpoint to within the
# precision of the kernel's scores, both neighbouring E4M3 codes are correct;
# the kernel's codes are read back (tattn_forward_dump) and admitted there
# only, then the oracle merges over them.

# Bound on the fp8 / fp4 MFMA's summation error relative to the sum of the
# products' magnitudes (measured at most 1.4e-4 for random E4M3 codes at
# K = 64; taken with margin).
MFMA_SUM_EPS = 2.5e-4
_DEC = None


def _e4m3_table():
    global _DEC
    if _DEC is None:
        from oracle import e4m3
        _DEC = e4m3.decode(np.arange(256, dtype=np.uint8))
    return _DEC


def _prow(m):
    """Place of staged key m's P value in the P.V operand order (bits 2 and 3
    of m swapped): with blocks of bk <= 8 keys, staged key m is key
    _prow(m) % bk of the step's block _prow(m) // bk (include/tattn.h,
    tattn_forward_dump)."""
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


# staged key of dump byte (half h, p): 32 (p / 16) + 8 ((p % 16) / 4) + 4 h + p % 4
_POS = np.arange(64)
_STAGED = 32 * ((_POS & 31) >> 4) + 8 * ((_POS & 15) >> 2) + 4 * (_POS >> 5) + (_POS & 3)


def quant_steps(counts_row, nk, bk, skim):
    """(LOW steps, SKIM steps) of one query block: a step holds one 64-key
    block or gathers 64 / bk smaller blocks of its tier."""
    nf, nl, ns = (int(x) for x in counts_row)
    g = 64 // bk
    nsk = nk - nf - nl - ns if skim else 0
    return -(-nl // g), -(-nsk // g)


def _staged(m, g, bk):
    """(slot, key) of staged key m of a step that gathers g blocks of bk keys."""
    if g == 1:
        return 0, m
    if g == 4:
        return m >> 4, m & 15
    return _prow(m) // bk, _prow(m) % bk


def kernel_tile_codes(dump_row, lists_row, counts_row, n, bq, bk, I, skim):
    """{J: uint8 [m_I, n_J]} codes of every LOW / SKIM tile of block I from its dump."""
    nk = lists_row.shape[0]
    nf, nl, ns = (int(x) for x in counts_row)
    g = 64 // bk
    m_i = min(bq, n - I * bq)
    sl, ssk = quant_steps(counts_row, nk, bk, skim)
    nsk = nk - nf - nl - ns if skim else 0
    out = {}
    # LOW steps first, then SKIM steps (tattn_forward_dump)
    for first, tiles, nsteps in ((0, lists_row[nf:nf + nl], sl), (sl, lists_row[nf + nl:nf + nl + nsk], ssk)):
        for s in range(nsteps):
            blocks = tiles[g * s: g * s + g]
            codes = dump_row[first + s, :m_i, :]                           # [m_I, 64] by dump byte
            for e in range(64):
                gi, key = _staged(_STAGED[e], g, bk)
                if gi >= len(blocks):
                    continue
                J = int(blocks[gi])
                nj = min(bk, n - J * bk)
                if key >= nj:
                    continue
                out.setdefault(J, np.zeros((m_i, nj), np.uint8))[:, key] = codes[:, e]
    return out


def admit_codes(kc, oc_codes, x, delta):
    """Kernel codes kc against the oracle's codes oc_codes of the same tile
    (x: the oracle's float32 value, delta: its relative error bound).  A code
    may differ from the oracle's only by one step and only where the midpoint
    between the two values lies within delta * x of x.  Returns (n_diff, n_bad)."""
    dec = _e4m3_table()
    diff = kc != oc_codes
    if not diff.any():
        return 0, 0
    a, b = kc[diff].astype(np.int64), oc_codes[diff].astype(np.int64)
    adjacent = (np.abs(a - b) == 1) & (a < 0x7F) & (b < 0x7F)
    mid = 0.5 * (dec[a] + dec[b])
    near = np.abs(x[diff] - mid) <= delta[diff] * x[diff] + 1e-30
    return int(diff.sum()), int((~(adjacent & near)).sum())


def tile_reference(oe, I, J, bq, bk, n, kind):
    """The oracle's scores, tile maximum, x, codes and the relative error bound
    of the kernel's x for one LOW or SKIM tile."""
    from oracle import tattn as T
    dec = _e4m3_table()
    d = oe["q8"].shape[1]
    r0, r1 = I * bq, min(n, (I + 1) * bq)
    j0, j1 = J * bk, min(n, (J + 1) * bk)
    if kind == T.LOW and oe.get("refine") is not None:
        # refined low tier: three products (T.refine_scores), each on the fp4 MFMA
        R = oe["refine"]
        q4, q4r, k4, k4r = R["q"][r0:r1], R["qr"][r0:r1], R["k"][j0:j1], R["kr"][j0:j1]
        scale = 1.0 / np.sqrt(d)
        s = T.refine_scores((q4, q4r), (k4, k4r)) * scale
        absum = T.refine_scores((np.abs(q4), np.abs(q4r)), (np.abs(k4), np.abs(k4r))) * scale
    else:
        if kind == T.LOW:
            qa, ka = dec[oe["q8"][r0:r1]], dec[oe["k8"][j0:j1]]
            scale = float(oe["sq"][I]) * float(oe["sk"][J]) / np.sqrt(d)
        else:
            qa, ka = oe["mx4"]["q"][r0:r1], oe["mx4"]["k"][j0:j1]
            scale = 1.0 / np.sqrt(d)
        s = (qa @ ka.T) * scale
        absum = (np.abs(qa) @ np.abs(ka).T) * scale                  # natural-log units
    mt, x, codes, _ = T.quantised_probabilities(s)
    l2e = 1.0 / np.log(2.0)
    # base-2 exponent error: MFMA sums of s_j and of the maximum, the float32
    # scale (two roundings) on s_j - m_t, the fused multiply-add, exp2
    dexp = (MFMA_SUM_EPS * (absum + absum.max(axis=1, keepdims=True)) * l2e
            + 3 * 2.0 ** -24 * np.abs(s - mt[:, None]) * l2e
            + 2.0 ** -23 * (np.abs(mt[:, None]) * l2e + 10.0) + 2.0 ** -22)
    delta = np.expm1(dexp * np.log(2.0)) + 2.0 ** -22
    return x, codes, delta


def admitted_codes(oe, tiers_row, lists_row, counts_row, dump_row, I, bq, bk, n, skim):
    """Kernel codes of block I's quantised tiles checked against the oracle's.
    Returns ({(I, J): codes}, n_codes, n_diff, n_bad)."""
    from oracle import tattn as T
    kcodes = kernel_tile_codes(dump_row, lists_row, counts_row, n, bq, bk, I, skim)
    want = set(np.nonzero((tiers_row == T.LOW) | (tiers_row == T.SKIM))[0].tolist())
    assert set(kcodes) == want, (I, sorted(set(kcodes) ^ want)[:8])
    out, tot, ndiff, nbad = {}, 0, 0, 0
    for J, kc in kcodes.items():
        x, oc, delta = tile_reference(oe, I, J, bq, bk, n, int(tiers_row[J]))
        dd, bb = admit_codes(kc, oc, x, delta)
        tot += kc.size
        ndiff += dd
        nbad += bb
        out[(I, J)] = kc
    return out, tot, ndiff, nbad


def forward_checked(tsm, p, dev, g, cfg, oc, rows=None, heads=None, out=None, log=print):
    """Forward through tattn_forward_dump, reading back the probability codes
    of the selected query blocks; each code is checked admissible against the
    oracle, and the oracle's output over the admitted codes is returned.
    rows: query blocks to compare (default all); heads: (b, h) pairs (default all).
    Returns (out numpy [B, H, N, d] float32, {(b, h): oracle output [N, d]
    (compared rows filled)}, {(b, h): rows})."""
    from oracle import tattn as T
    tiers = p.tiers()
    lists, counts = p.lists()
    nq, nk = cfg.n_qblocks, cfg.n_kblocks
    skim = p.cfg.tau_skim > 0 and int(p.cfg.mode) != 2     # every routed mode has the SKIM tier then
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)] if heads is None else heads
    sel = []
    for (b, h) in heads:
        rr = list(range(nq)) if rows is None else (rows(b, h, tiers[b, h]) if callable(rows) else rows)
        sel += [(b, h, int(I)) for I in rr]
    steps = max([sum(quant_steps(counts[b, h, I], nk, cfg.block_k, skim)) for (b, h, I) in sel] + [1])
    o, dump = tsm.forward_dump(p, dev["q"], dev["k"], dev["v"], sel, steps, out=out)
    o = o.float().cpu().numpy()
    refs, used = {}, {}
    tot = ndiff = nbad = 0
    for (b, h) in heads:
        mine = [(i, I) for i, (bb, hh, I) in enumerate(sel) if (bb, hh) == (b, h)]
        q, k, v = g["q"][b, h], g["k"][b, h], g["v"][b, h]
        oe = T.oracle_plan(q, k, v, oc, mode=3, external_tiers=tiers[b, h])
        codes = {}
        for i, I in mine:
            c, t_, d_, b_ = admitted_codes(oe, tiers[b, h, I], lists[b, h, I], counts[b, h, I], dump[i], I,
                                           cfg.block_q, cfg.block_k, cfg.seq_len, skim)
            codes.update(c)
            tot, ndiff, nbad = tot + t_, ndiff + d_, nbad + b_
        rws = [I for _, I in mine]
        refs[(b, h)] = T.oracle_forward(q, k, v, oe, cfg.block_q, cfg.block_k, rows=rws, p_codes=codes)
        used[(b, h)] = rws
    log(f"  probability codes: {tot} checked, {ndiff} differ from the oracle's "
        f"({(ndiff / max(tot, 1)):.2e}), {nbad} outside the admissible band")
    assert nbad == 0, (nbad, ndiff, tot)
    return o, refs, used


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64."""
    from synth.gen import to_bf16_bits, bf16_bits_to_f32
    return bf16_bits_to_f32(to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))).astype(np.float64)


def check_forward(tsm, p, dev, g, cfg, oc, rows=None, heads=None, what="", log=print):
    """The forward of plan p against the oracle under p's tier map: the
    kernel's probability codes admitted (forward_checked), then per compared
    query block max-abs <= 1e-2 and mean-abs <= 1e-3 against the oracle.
    With bfloat16 output the output carries one more rounding: max-abs <= 1e-2
    plus half a bfloat16 ulp of the oracle's value, and mean-abs <= 1e-3
    against the oracle rounded to bfloat16.  Returns (out, refs)."""
    o, refs, used = forward_checked(tsm, p, dev, g, cfg, oc, rows=rows, heads=heads, log=log)
    bf16 = int(p.cfg.out_dtype) == 0
    worst_max = worst_mean = 0.0
    for (b, h), ref in refs.items():
        for I in used[(b, h)]:
            r0, r1 = I * cfg.block_q, min(cfg.seq_len, (I + 1) * cfg.block_q)
            got, want = o[b, h, r0:r1].astype(np.float64), ref[r0:r1]
            err = np.abs(got - want)
            if bf16:
                # half an ulp of bfloat16 (8 significant bits) at |want|
                half_ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 9)
                over = float((err - half_ulp).max())
                mean = float(np.abs(got - bf16_round(want)).mean())
            else:
                over, mean = float(err.max()), float(err.mean())
            worst_max, worst_mean = max(worst_max, over), max(worst_mean, mean)
            assert over <= 1e-2 and mean <= 1e-3, (what, b, h, I, over, mean)
    log(f"  {what}: worst block max-abs {worst_max:.3e} mean-abs {worst_mean:.3e}"
        f"{' (bf16 output: max-abs beyond half a bf16 ulp; mean-abs against the oracle rounded to bf16)' if bf16 else ''}")
    return o, refs


# ---- full-size launches from a few generated heads tiled to the full head count
def sample_rows(nq, n, tiers):
    """n query blocks: the first and the ragged last, the rows with the most
    LOW tiles and with the most FULL tiles (a quarter of n each), then evenly
    spaced ones."""
    rows = [0, nq - 1]
    for tier in (1, 2):
        added = 0
        for I in np.argsort(-(tiers == tier).sum(axis=1), kind="stable"):
            if added >= n // 4 or len(rows) >= n:
                break
            if int(I) not in rows:
                rows.append(int(I))
                added += 1
    for I in np.linspace(0, nq - 1, n).astype(int):
        if len(rows) >= min(n, nq):
            break
        if int(I) not in rows:
            rows.append(int(I))
    return sorted(rows)


def device_tiled(bits, heads):
    import torch
    out = {}
    for n in ("q", "k", "v"):
        t = torch.from_numpy(bits[n].view(np.int16)).view(torch.bfloat16).cuda()
        idx = torch.arange(heads, device="cuda") % t.shape[1]
        out[n] = t.index_select(1, idx).contiguous()
    return out


class TiledHeads:
    """The generated heads seen at the tiled head indices."""

    def __init__(self, g, gen_heads):
        self.g, self.n = g, gen_heads

    def __getitem__(self, name):
        x = self.g[name]
        return HeadView(x, self.n)


class HeadView:
    def __init__(self, x, n):
        self.x, self.n = x, n

    def __getitem__(self, idx):
        b, h = idx
        return self.x[b, h % self.n]
