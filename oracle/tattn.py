"""Three-tier tile-sparse attention, computed plainly on the CPU -- TEST
INFRASTRUCTURE ONLY (tests, smoke check and the bench's cpu_baseline leg).

Per (batch, head) the method runs four steps; each function below names the
passage it follows.  Notation: N tokens, head dim d, query blocks I of Bq rows
(m_I real rows), key blocks J of Bk keys (n_J real keys); the last blocks are
ragged and keep their real sizes.

  O1/O2 pool        q_I, k_J, v_J block means            (Triage: block means;
                                                          HierPAS: lightweight
                                                          eager estimate)
  O3    router      p_IJ = softmax_J(q_I.k_J/sqrt(d) + ln n_J)
                                                         (APT: attention
                                                          probability as the
                                                          importance metric)
  O4    tiers       dual thresholds tau_hi / tau_lo, optional top-k, or the
                    entropy-derived head-adaptive top-k, or the price router
                    (predicted per-tier error from block second moments
                    against one price); diagonal tiles FULL
                                                         (APT: dual
                                                          thresholds; HierPAS:
                                                          top-k and head-wise
                                                          retention ratios;
                                                          Triage: error-
                                                          predicting router)
  O5    fp8         E4M3 codes with one scale per block   (HierPAS: reduced
                                                          precision); a low
                                                          tile runs attention
                                                          on these copies
  O6/O7 attention   per-tile partials (m, l, o) for FULL / LOW / SKIP tiles,
                    merged exactly                        (Triage: skip =
                                                          block means, one
                                                          fused pass)

A low-precision tile (LOW, and the 4-bit SKIM tier) runs its whole tile on
8-bit operands: scores from the E4M3 (or MXFP4) copies of q and k, the tile's
probabilities quantised to E4M3 against the tile-local row maximum
(pi_j = decode(E(fl32(448 e^{s_j - m_t}))) / 448, so the maximum lands on 448
exactly and a tile's codes do not depend on the order tiles are visited in),
values from the E4M3 copy of V, v^ = fl32(decode(code) * scale); the tile's
share of the row normaliser sums the same pi (HierPAS: progressively reduced
precision; APT: dual-precision execution).  In the refine variant of the low
tier the scores come from MXFP4 copies with an MXFP4 residual correction
(Triage: refining a tile with 4-bit residual correction; refine_operands).

Precision: float64 throughout, except that every fp8 code is decided on a
float32 value (a code is an integer decided by a floating-point value, and
that decision is taken in float32 wherever it is made) and the dequantised
E4M3 values are products rounded once to float32.  Means are accumulated in float64 and
stored as float32.
"""
import math

import numpy as np

from . import e4m3, mxfp4

SKIP, LOW, FULL, SKIM = 0, 1, 2, 3

LOG2E = 1.0 / math.log(2.0)


# ----------------------------------------------------------------------------- O1
def block_sizes(n: int, b: int) -> np.ndarray:
    """Real sizes of the ceil(n/b) contiguous blocks of b tokens (last one ragged).
    Blocks are contiguous runs of the row-major (t, h, w) token order."""
    nb = -(-n // b)
    sizes = np.full(nb, b, dtype=np.int64)
    sizes[-1] = n - (nb - 1) * b
    return sizes


# ----------------------------------------------------------------------------- O2
def pool_means(x: np.ndarray, b: int) -> np.ndarray:
    """Block means of x [n, d]: float64 sum divided by the real block size,
    rounded to float32 (Triage: a skipped tile is replaced by its block means;
    HierPAS: a lightweight estimate of the attention pattern)."""
    n, d = x.shape
    sizes = block_sizes(n, b)
    out = np.empty((sizes.size, d), dtype=np.float32)
    x64 = x.astype(np.float64)
    for j, s in enumerate(sizes):
        blk = x64[j * b: j * b + s]
        out[j] = (blk.sum(axis=0) / float(s)).astype(np.float32)
    return out


# ----------------------------------------------------------------------------- O3
def router(qbar: np.ndarray, kbar: np.ndarray, n: int, bk: int):
    """Block router: S_IJ = <q_I, k_J>/sqrt(d) + ln n_J and p_IJ = softmax over J
    (APT: attention probabilities rank the tiles; the ln n_J term makes p_IJ the
    block's share of attention mass when every key of J equals k_J).
    Returns (S, p) in float64, shape [Nq, Nk]."""
    d = qbar.shape[1]
    nk = block_sizes(n, bk).astype(np.float64)
    S = (qbar.astype(np.float64) @ kbar.astype(np.float64).T) / math.sqrt(d) + np.log(nk)[None, :]
    mx = S.max(axis=1, keepdims=True)
    e = np.exp(S - mx)
    p = e / e.sum(axis=1, keepdims=True)
    return S, p


# ----------------------------------------------------------------------------- O4
def diagonal_mask(n: int, bq: int, bk: int) -> np.ndarray:
    """Tiles whose key-token range intersects the query block's token range
    ("the diagonal block is always full"); with bq != bk a row has several."""
    nq, nk = -(-n // bq), -(-n // bk)
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        r0, r1 = i * bq, min(n, (i + 1) * bq)
        j0, j1 = r0 // bk, (r1 - 1) // bk
        m[i, j0:j1 + 1] = True
    return m


def row_ranks(p: np.ndarray) -> np.ndarray:
    """Rank of every tile within its row by (p descending, J ascending)."""
    nq, nk = p.shape
    ranks = np.empty((nq, nk), dtype=np.int64)
    cols = np.arange(nk)
    for i in range(nq):
        order = np.lexsort((cols, -p[i]))
        ranks[i, order] = cols
    return ranks


def tiers_threshold(p: np.ndarray, tau_hi: float, tau_lo: float, top_k: int = 0,
                    tau_skim: float = 0.0) -> np.ndarray:
    """Dual thresholds on the router probability (APT's dual thresholding at
    tile granularity): FULL if p >= tau_hi, LOW if tau_lo <= p < tau_hi, SKIP
    below tau_lo.  With tau_skim > 0 a third threshold splits the band below
    tau_lo: SKIM (the 4-bit tier, Triage's skimming) if tau_skim <= p < tau_lo.
    With top_k > 0 only a row's top_k tiles (HierPAS: top-k) may be kept;
    thresholds then act inside them.  Diagonal forcing is separate."""
    t = np.full(p.shape, SKIP, dtype=np.uint8)
    if tau_skim > 0:
        t[p >= tau_skim] = SKIM
    t[p >= tau_lo] = LOW
    t[p >= tau_hi] = FULL
    if top_k > 0:
        t[row_ranks(p) >= top_k] = SKIP
    return t


def head_retention(p: np.ndarray, samples: int, keep_min: float, keep_max: float):
    """Sampling-based entropy -> head-wise retention ratio (HierPAS).  Rows
    I_s = floor(s*Nq/S), s < S = min(samples, Nq); H_I = -sum_J p ln p;
    r_h = clip(exp(mean_s H)/Nk, keep_min, keep_max) (the perplexity share of
    key blocks); k_h = ceil(r_h * Nk).  The exp(mean entropy)/Nk mapping is a
    reading of the pages, which give no formula: parity unpinned."""
    nq, nk = p.shape
    S = min(samples, nq)
    rows = (np.arange(S) * nq) // S
    P = p[rows]
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0, P * np.log(P), 0.0)
    H = -plogp.sum(axis=1)
    r = float(np.clip(math.exp(float(H.mean())) / nk, keep_min, keep_max))
    k = int(math.ceil(r * nk))
    return r, k, H


def tiers_adaptive(p: np.ndarray, k_h: int, full_frac: float, tau_skim: float = 0.0) -> np.ndarray:
    """Head-adaptive tiers: per row, the k_h highest-p tiles are kept; the top
    ceil(full_frac * k_h) of them run in bf16 (FULL), the rest of the kept ones
    in fp8 (LOW), the remainder is skipped.  With tau_skim > 0 (Triage's 4-bit
    skim tier, reading R18) a tile outside the kept ones is SKIM when
    p >= tau_skim (float32 tau widened to float64)."""
    ranks = row_ranks(p)
    nfull = int(math.ceil(full_frac * k_h))
    t = np.full(p.shape, SKIP, dtype=np.uint8)
    t[ranks < k_h] = LOW
    t[ranks < nfull] = FULL
    if tau_skim > 0:
        t[(t == SKIP) & (p >= float(np.float32(tau_skim)))] = SKIM
    return t


# ----------------------------------------------------------------------------- O4b price router
# Triage's router predicts, from block statistics, the output error a tile
# would incur under each tier and moves it to a more accurate tier only when
# the predicted error reduction is worth the extra compute at one price.  The
# pages give no formula; the model below is this implementation's reading
# (parity unpinned as a predictor; its exact identities are pinned).

E4M3_U = 2.0 ** -4          # largest relative rounding error of an E4M3 normal value
MXFP4_U = 2.0 ** -2         # largest relative rounding error of an E2M1 normal value
# bf16-equivalent MFMA work per tile, at the matrix rates (fp8 twice, fp4 four
# times the bf16 rate): LOW = fp8 scores + fp8 P.V; SKIM = fp4 scores + fp8 P.V
COST_FULL, COST_LOW = 1.0, 0.5
COST_SKIM = 0.375


def cost_skip(bk: int) -> float:
    """Work of a skipped block relative to a FULL tile of the same shape: one
    pseudo-key scored twice (bf16 hi + lo parts of k_J) plus its P.V share."""
    return 1.5 / bk


def block_moments(x: np.ndarray, b: int):
    """Second-moment statistics of each block of b rows (real size s), from
    float64 sums S1_c = sum_i x_ic and S2_c = sum_i x_ic^2:
      m2[j, c]  = S2_c / s                         (mean square per dimension)
      var[j, c] = max(S2_c / s - (S1_c / s)^2, 0)  (variance per dimension)
      tot_m2[j] = sum_c m2, tot_var[j] = sum_c var, mnorm[j] = sqrt(sum_c (S1_c / s)^2)
    every output rounded once to float32."""
    n, d = x.shape
    sizes = block_sizes(n, b)
    nb = sizes.size
    m2 = np.empty((nb, d), np.float32)
    var = np.empty((nb, d), np.float32)
    tot_m2 = np.empty(nb, np.float32)
    tot_var = np.empty(nb, np.float32)
    mnorm = np.empty(nb, np.float32)
    x64 = x.astype(np.float64)
    for j, sz in enumerate(sizes):
        blk = x64[j * b: j * b + sz]
        mean = blk.sum(axis=0) / float(sz)
        msq = (blk * blk).sum(axis=0) / float(sz)
        vr = np.maximum(msq - mean * mean, 0.0)
        m2[j], var[j] = msq.astype(np.float32), vr.astype(np.float32)
        tot_m2[j], tot_var[j] = np.float32(msq.sum()), np.float32(vr.sum())
        mnorm[j] = np.float32(math.sqrt(float((mean * mean).sum())))
    return dict(m2=m2, var=var, tot_m2=tot_m2, tot_var=tot_var, mnorm=mnorm)


def tile_error_model(q2, m2q, kvar, m2k, vvar, m2v, vnorm, n_k, d, skim=False):
    """Predicted relative output error of every tile (I, J) under SKIP and LOW
    (FULL: 0), float64 [Nq, Nk] each.  Inputs are the float32 block statistics
    of block_moments (q2 = query m2 per dimension, m2q its total; kvar = key
    variance per dimension, m2k the key mean square total; vvar, m2v, vnorm =
    value variance total, mean square total and mean norm) and the real key
    block sizes n_k.

    Within a tile a key's score deviates from the pooled score by
    delta = q_i.(k_j - k_J)/sqrt(d); over the tile's (query, key) pairs its
    mean square, taking the dimensions as uncorrelated, is
        s2 = sum_c q2[I, c] kvar[J, c] / d.
    The weights e^delta are taken as lognormal.  The block's mass then exceeds
    the pooled estimate n_J e^S by the log-gain
        g = s2/2                        (s2 <= 2 ln n_J: the lognormal mean)
        g = sqrt(2 s2 ln n_J) - ln n_J  (beyond: the largest of n_J scores
                                         dominates the sum)
    and the weights keep n_eff = max(1, n_J e^-s2) keys' worth of values.
      SKIP  (block means, one score weighted by n_J): the mass falls short by
            the factor e^-g and the block-mean value misses the weighted mean:
            eS = vnorm (1 - e^-g) + sqrt(vvar max(0, 1/n_eff - 1/n_J)).
      LOW   (E4M3 copies of q, k, v): rounding errors of relative RMS u/sqrt(3)
            add score noise of variance sl2 = (2u^2/3) m2q m2k / d^2 and value
            noise of RMS u sqrt(m2v/3):
            eL = vnorm expm1(sl2/2)
                 + (sqrt(vvar expm1(sl2)) + u sqrt(m2v/3)) / sqrt(n_eff).
      SKIM  (MXFP4 scores, with skim=True): the same form with E2M1's bound
            u = 2^-2 in place of E4M3's 2^-4 in the score noise sk2 (its
            rounding is relative to the 32-element block's scale, and the
            relative bound covers it); its values are E4M3 as in LOW.
    The norm of the block mean stands in for the distance between the tile's
    output and the row's.  Returns (s2, g, eS, eL), and eK after them with
    skim=True."""
    q2 = q2.astype(np.float64)
    kvar = kvar.astype(np.float64)
    s2 = (q2 @ kvar.T) / d                                              # [Nq, Nk]
    sl2 = (2.0 * E4M3_U ** 2 / 3.0) * np.outer(m2q.astype(np.float64), m2k.astype(np.float64)) / float(d * d)
    nj = n_k.astype(np.float64)[None, :]
    lnn = np.log(nj)
    g = np.where(s2 <= 2.0 * lnn, 0.5 * s2, np.sqrt(2.0 * s2 * lnn) - lnn)
    neff = np.maximum(1.0, nj * np.exp(-s2))
    vn = vnorm.astype(np.float64)[None, :]
    vv = vvar.astype(np.float64)[None, :]
    mv = m2v.astype(np.float64)[None, :]
    eS = vn * (-np.expm1(-g)) + np.sqrt(vv * np.maximum(0.0, 1.0 / neff - 1.0 / nj))
    eL = vn * np.expm1(0.5 * sl2) + (np.sqrt(vv * np.expm1(sl2)) + E4M3_U * np.sqrt(mv / 3.0)) / np.sqrt(neff)
    if not skim:
        return s2, g, eS, eL
    sk2 = (2.0 * MXFP4_U ** 2 / 3.0) * np.outer(m2q.astype(np.float64), m2k.astype(np.float64)) / float(d * d)
    eK = vn * np.expm1(0.5 * sk2) + (np.sqrt(vv * np.expm1(sk2)) + E4M3_U * np.sqrt(mv / 3.0)) / np.sqrt(neff)
    return s2, g, eS, eL, eK


def corrected_shares(S: np.ndarray, g: np.ndarray) -> np.ndarray:
    """The router's row softmax with every tile's log-mass raised by its
    spread gain g: p~_IJ = softmax_J(S_IJ + g_IJ), float64."""
    x = S + g
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def tiers_price(p: np.ndarray, eS: np.ndarray, eL: np.ndarray, price: float, bk: int, eK=None):
    """Each tile takes the tier t minimising p_IJ * e_t + price * cost_t, i.e.
    it moves to a more accurate tier only when the predicted error reduction
    (the relative error scaled by the tile's share p of the row) pays for the
    extra work at the given price (Triage: one price sets the trade-off).
    With eK the SKIM tier is a fourth choice (Triage: skip, skim in 4 bits,
    refine).  Ties go to the cheaper tier (SKIP < SKIM < LOW < FULL in work).
    Returns the tier map and the objectives (SKIP, LOW, FULL, then SKIM)."""
    lam = float(price)
    oS = p * eS + lam * cost_skip(bk)
    oL = p * eL + lam * COST_LOW
    oF = np.full(p.shape, lam * COST_FULL)
    t = np.full(p.shape, SKIP, dtype=np.uint8)
    best = oS.copy()
    if eK is not None:
        oK = p * eK + lam * COST_SKIM
        t[oK < best] = SKIM
        best = np.minimum(best, oK)
    t[oL < best] = LOW
    best = np.minimum(best, oL)
    t[oF < best] = FULL
    return t, ((oS, oL, oF) if eK is None else (oS, oL, oF, oK))


def build_lists(t: np.ndarray):
    """Per query block: kept/skipped key-block indices, [FULL asc | LOW asc |
    SKIM asc | SKIP asc], and the counts of FULL, LOW and SKIP (the SKIM count
    is the rest of the row) (APT's mask management, as compacted lists)."""
    nq, nk = t.shape
    lists = np.empty((nq, nk), dtype=np.int16)
    counts = np.empty((nq, 3), dtype=np.int32)
    for i in range(nq):
        f = np.nonzero(t[i] == FULL)[0]
        lo = np.nonzero(t[i] == LOW)[0]
        k4 = np.nonzero(t[i] == SKIM)[0]
        s = np.nonzero(t[i] == SKIP)[0]
        lists[i] = np.concatenate([f, lo, k4, s]).astype(np.int16)
        counts[i] = (f.size, lo.size, s.size)
    return lists, counts


# ----------------------------------------------------------------------------- O5
def quantise_blocks(x: np.ndarray, b: int):
    """fp8 E4M3 codes with one scale per block of b rows (HierPAS: reduced
    precision for less critical regions).  a = max|X_block| (float32);
    a == 0 -> inv = scale = 1; else inv = fl32(448/a), scale = fl32(a/448);
    code = E(fl32(x * inv)).  Returns (codes uint8 [n, d], scale f32, inv f32)."""
    n, d = x.shape
    x32 = x.astype(np.float32)
    sizes = block_sizes(n, b)
    scale = np.empty(sizes.size, dtype=np.float32)
    inv = np.empty(sizes.size, dtype=np.float32)
    codes = np.empty((n, d), dtype=np.uint8)
    for j, s in enumerate(sizes):
        blk = x32[j * b: j * b + s]
        a = np.float32(np.abs(blk).max())
        if a == 0:
            iv, sc = np.float32(1.0), np.float32(1.0)
        else:
            iv, sc = np.float32(448.0) / a, a / np.float32(448.0)
        inv[j], scale[j] = iv, sc
        codes[j * b: j * b + s] = e4m3.encode((blk * iv).astype(np.float32))
    return codes, scale, inv


def skim_operands(q, k):
    """Score operands of skim tiles (Triage: skimming a tile in a 4-bit
    format): Q and K each quantised to MXFP4 per token row, one E8M0 scale per
    32 consecutive channels; the scores use the dequantised values exactly.
    (A skim tile's probabilities and values are those of the low tier: see
    quantised_probabilities.)  Returns a dict of the dequantised operands
    (float64 [n, d]) and the codes and scale bytes of k."""
    _, _, qd = mxfp4.quantise(q)
    kc, ks, kd = mxfp4.quantise(k)
    return dict(q=qd, k=kd, k_codes=kc, k_scales=ks)


def refine_operands(q, k):
    """Score operands of the residual-corrected refine variant of the low tier
    (Triage: a tile refined with 4-bit residual correction).  Each of Q and K
    is quantised to MXFP4 per token row (one E8M0 scale per 32 channels), and
    the rounding residual x - x4 is quantised to MXFP4 again with its own
    scales: x ~ x4 + x4r.  A tile's scores keep the three products of order
    up to one in the residuals, <q4, k4> + <q4, k4r> + <q4r, k4> (over
    sqrt(d)); the product of the two residuals is of second order and dropped
    (reading R20).  Returns the dequantised operands (float64 [n, d]) and the
    codes and scale bytes of k and of its residual."""
    _, _, qd = mxfp4.quantise(q)
    _, _, qrd = mxfp4.quantise(np.asarray(q, np.float64) - qd)
    kc, ks, kd = mxfp4.quantise(k)
    krc, krs, krd = mxfp4.quantise(np.asarray(k, np.float64) - kd)
    return dict(q=qd, qr=qrd, k=kd, kr=krd, k_codes=kc, k_scales=ks, kr_codes=krc, kr_scales=krs)


def refine_scores(qa, ka):
    """Unscaled refine scores of query rows against key rows: with qa = (q4,
    q4r) and ka = (k4, k4r), <q4, k4> + <q4, k4r> + <q4r, k4>."""
    q4, q4r = qa
    k4, k4r = ka
    return q4 @ k4.T + q4 @ k4r.T + q4r @ k4.T


def dequantise(codes: np.ndarray, scale: np.ndarray, b: int) -> np.ndarray:
    """X^ = fl32(decode(code) * scale) with the scale of each row's block of b
    rows.  Returns float64 [n, d] (values representable in float32)."""
    n = codes.shape[0]
    blk = np.repeat(np.arange(-(-n // b)), b)[:n]
    return (e4m3.decode(codes).astype(np.float32) * scale.astype(np.float32)[blk][:, None]).astype(np.float64)


P_MAX = 448.0   # E4M3's largest finite value: the tile maximum's probability code


def quantised_probabilities(s: np.ndarray):
    """Probabilities of a low-precision tile (HierPAS: reduced precision for
    less critical tiles), quantised to E4M3 against the tile-local row maximum:
      m_t  = max_j s_j over the tile's keys (per query row; s float64, -inf
             marks a key past the end of the sequence),
      x_j  = fl32(448 e^{s_j - m_t})            (the maximum lands on 448),
      c_j  = E(x_j)                             (round to nearest even),
      pi_j = decode(c_j) / 448.
    s: [..., n] scores of one tile per leading index.  Returns (m_t, x, c, pi)
    with x float64 (float32 values), c uint8 and pi float64."""
    mt = s.max(axis=-1)
    x = (P_MAX * np.exp(s - mt[..., None])).astype(np.float32).astype(np.float64)
    c = e4m3.encode(x)
    return mt, x, c, e4m3.decode(c) / P_MAX


def low_scores(qc: np.ndarray, sq: float, kc: np.ndarray, sk: float, d: int) -> np.ndarray:
    """Scores of a LOW tile from the E4M3 copies: s^_ij = <q^_i, k^_j>/sqrt(d)
    with q^ = decode(q8) sq and k^ = decode(k8) sk taken exactly (float64).
    qc: [m, d] and kc: [n, d] decoded code values."""
    return (qc @ kc.T) * (float(sq) * float(sk) / math.sqrt(d))


# ----------------------------------------------------------------------------- O6/O7
def _padded(x, nb, b):
    n, d = x.shape
    out = np.zeros((nb * b, d), dtype=np.float64)
    out[:n] = x
    return out.reshape(nb, b, d)


def attention_forward(q, k, v, t, bq, bk, kbar, vbar, q8, sq, k8, sk, v8, sv,
                      rows=None, return_partials=False, mx4=None, p_codes=None, refine=None):
    """One pass over all tiles of every query row, merging per-tile partials
    exactly (Triage: skip, low precision and full tiles in a single pass).

    FULL: s_j = <q_i,k_j>/sqrt(d); partial (max s, sum e^{s-m}, sum e^{s-m} v_j).
    LOW:  scores s^_j from the E4M3 copies (low_scores), probabilities
          quantised against the tile max (quantised_probabilities), values
          v^_j = fl32(decode(V8_j) * sv_J); partial (m_t, sum pi_j, sum pi_j v^_j).
          With ``refine`` (refine_operands) a LOW tile's scores are instead
          <q4,k4> + <q4,k4r> + <q4r,k4> over sqrt(d) (refine_scores).
    SKIM: the same with scores from the MXFP4 copies (``mx4``, skim_operands):
          <q4_i, k4_j>/sqrt(d) (Triage: skimming in 4 bits); probabilities and
          values as in LOW.
    SKIP: sigma = <q_i, k_J>/sqrt(d) + ln n_J; partial (sigma, 1, v_J): one
          score weighted by n_J, valued by the block mean (Triage).
    Merge: M = max m; O_i = sum o e^{m-M} / sum l e^{m-M}.

    q, k, v: [n, d] (values as float64); t: tier map [Nq, Nk].
    ``rows`` restricts the computation to those query blocks (others left 0).
    ``p_codes``: optional {(I, J): uint8 [m_I, n_J]} probability codes used in
    place of the quantised ones for those LOW / SKIM tiles (a tile's codes are
    not unique where x_j lies on a rounding midpoint to within the precision
    of its scores; the caller decides which codes are admissible).
    Returns O float64 [n, d] (and the per-row partial lists if requested)."""
    n, d = q.shape
    nq, nk = t.shape
    isd = 1.0 / math.sqrt(d)
    ksz = block_sizes(n, bk)
    valid = np.arange(bk)[None, :] < ksz[:, None]                      # [Nk, Bk]
    Kp = _padded(k.astype(np.float64), nk, bk)
    Vp = _padded(v.astype(np.float64), nk, bk)
    Kh = _padded(e4m3.decode(k8), nk, bk)                              # code values
    Vh = _padded(dequantise(v8, sv, bk), nk, bk)
    Qc = e4m3.decode(q8)
    if np.any(t == SKIM):
        Kq = _padded(mx4["k"], nk, bk)
    if refine is not None:
        Kr4, Kr4r = _padded(refine["k"], nk, bk), _padded(refine["kr"], nk, bk)
    kb64, vb64 = kbar.astype(np.float64), vbar.astype(np.float64)
    lnk = np.log(ksz.astype(np.float64))
    out = np.zeros((n, d), dtype=np.float64)
    partials = {}

    def quantised_partial(i, Js, s):
        """(m_t, sum pi, sum pi v^) of the quantised tiles Js of row i; s [m, nJ, bk]."""
        mt, _, c, pi = quantised_probabilities(np.where(valid[Js][None], s, -np.inf))
        if p_codes is not None:
            for a, J in enumerate(Js):
                if (i, int(J)) in p_codes:
                    c[:, a, :] = 0
                    cc = np.asarray(p_codes[(i, int(J))], np.uint8)
                    c[:, a, :cc.shape[1]] = cc
                    pi[:, a, :] = e4m3.decode(c[:, a, :]) / P_MAX
        pi = np.where(valid[Js][None], pi, 0.0)
        return mt, pi.sum(axis=2), np.matmul(pi.transpose(1, 0, 2), Vh[Js]).transpose(1, 0, 2)

    for i in (range(nq) if rows is None else rows):
        r0, r1 = i * bq, min(n, (i + 1) * bq)
        Q = q[r0:r1].astype(np.float64)
        ms, ls, os_ = [], [], []
        F = np.nonzero(t[i] == FULL)[0]
        if F.size:
            s = (Q @ Kp[F].reshape(-1, d).T).reshape(r1 - r0, F.size, bk) * isd
            s = np.where(valid[F][None], s, -np.inf)
            m = s.max(axis=2)
            e = np.exp(s - m[..., None])
            ms.append(m)
            ls.append(e.sum(axis=2))
            os_.append(np.matmul(e.transpose(1, 0, 2), Vp[F]).transpose(1, 0, 2))
        L = np.nonzero(t[i] == LOW)[0]
        if L.size and refine is not None:
            s = refine_scores((refine["q"][r0:r1], refine["qr"][r0:r1]),
                              (Kr4[L].reshape(-1, d), Kr4r[L].reshape(-1, d)))
            m, l, o = quantised_partial(i, L, s.reshape(r1 - r0, L.size, bk) * isd)
            ms.append(m)
            ls.append(l)
            os_.append(o)
        elif L.size:
            raw = (Qc[r0:r1] @ Kh[L].reshape(-1, d).T).reshape(r1 - r0, L.size, bk)
            sc = float(sq[i]) * sk.astype(np.float64)[L] * isd            # [nL]
            m, l, o = quantised_partial(i, L, raw * sc[None, :, None])
            ms.append(m)
            ls.append(l)
            os_.append(o)
        K4 = np.nonzero(t[i] == SKIM)[0]
        if K4.size:
            s = (mx4["q"][r0:r1] @ Kq[K4].reshape(-1, d).T).reshape(r1 - r0, K4.size, bk) * isd
            m, l, o = quantised_partial(i, K4, s)
            ms.append(m)
            ls.append(l)
            os_.append(o)
        Sk = np.nonzero(t[i] == SKIP)[0]
        skip_sigma = None
        if Sk.size:
            skip_sigma = Q @ kb64[Sk].T * isd + lnk[Sk][None, :]          # [m, nS]
        # merge (O7)
        allm = [x for x in ms] + ([skip_sigma] if skip_sigma is not None else [])
        M = np.max(np.concatenate(allm, axis=1), axis=1)                   # [m]
        num = np.zeros((r1 - r0, d))
        den = np.zeros(r1 - r0)
        for m, l, o in zip(ms, ls, os_):
            w = np.exp(m - M[:, None])
            den += (w * l).sum(axis=1)
            num += np.einsum("it,itd->id", w, o)
        if skip_sigma is not None:
            w = np.exp(skip_sigma - M[:, None])
            den += w.sum(axis=1)
            num += w @ vb64[Sk]
        out[r0:r1] = num / den[:, None]
        if return_partials:
            partials[i] = (ms, ls, os_, skip_sigma, M, den)
    if return_partials:
        return out, partials
    return out


def effective_weights(q, k, v, t, bq, bk, kbar, q8, sq, k8, sk, v8, sv, mx4=None):
    """Dense [n, n] weight matrix W of the method on tiny inputs, together with
    the value matrix each weight multiplies, built one query row and one tile
    at a time with scalar bookkeeping:
      FULL  w_j = e^{s_j - M} against v_j,
      LOW   w_j = pi_j e^{m_t - M} against v^_j (scores from the E4M3 copies),
      SKIM  the same with scores from the MXFP4 copies,
      SKIP  w_j = e^{sigma - M} / n_J for every j in J, against v_j,
    with M the largest of the row's FULL scores, LOW / SKIM tile maxima and
    SKIP scores, and W = w / sum w.  Then O = rowsum(W * Vsel)."""
    n, d = q.shape
    nq, nk = t.shape
    isd = 1.0 / math.sqrt(d)
    ksz = block_sizes(n, bk)
    qblk = np.repeat(np.arange(nq), bq)[:n]
    khat = e4m3.decode(k8)
    vhat = dequantise(v8, sv, bk)
    qc = e4m3.decode(q8)
    W = np.zeros((n, n))
    sel_q = np.zeros((n, n), dtype=bool)
    for i in range(n):
        I = qblk[i]
        refs, terms = [], []          # per tile: (reference m, list of (j, factor))
        for J in range(nk):
            j0, j1 = J * bk, J * bk + ksz[J]
            tier = t[I, J]
            if tier == FULL:
                s = (k[j0:j1].astype(np.float64) @ q[i].astype(np.float64)) * isd
                m = float(s.max())
                refs.append(m)
                terms.append([(j0 + a, math.exp(float(s[a]) - m)) for a in range(j1 - j0)])
            elif tier == SKIP:
                sig = float(q[i].astype(np.float64) @ kbar[J].astype(np.float64)) * isd + math.log(ksz[J])
                refs.append(sig)
                terms.append([(j0 + a, 1.0 / ksz[J]) for a in range(j1 - j0)])
            else:
                if tier == SKIM:
                    s = (mx4["k"][j0:j1] @ mx4["q"][i]) * isd
                else:
                    s = low_scores(qc[i:i + 1], sq[I], khat[j0:j1], sk[J], d)[0]
                m, _, _, pi = quantised_probabilities(s)
                refs.append(float(m))
                terms.append([(j0 + a, float(pi[a])) for a in range(j1 - j0)])
                sel_q[i, j0:j1] = True
        M = max(refs)
        for m, tl in zip(refs, terms):
            f = math.exp(m - M)
            for j, w in tl:
                W[i, j] = w * f
        W[i] /= W[i].sum()
    vsel = np.where(sel_q[:, :, None], vhat[None, :, :], v[None, :, :].astype(np.float64))
    return W, vsel


def naive_attention(q, k, v):
    """Textbook softmax(Q K^T / sqrt(d)) V in float64."""
    d = q.shape[1]
    s = q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


# ----------------------------------------------------------------------------- whole plan / forward
def oracle_plan(q, k, v, cfg_like, mode=None, external_tiers=None):
    """Steps O1-O5 for one (batch, head): q, k, v [n, d].  ``cfg_like`` needs
    block_q, block_k, tau_hi, tau_lo, top_k, mode, keep_min, keep_max,
    full_frac, entropy_samples (and price for mode 4, the price router).
    Returns a dict of every intermediate."""
    mode = cfg_like.mode if mode is None else mode
    n, d = q.shape
    bq, bk = cfg_like.block_q, cfg_like.block_k
    qbar = pool_means(q, bq)
    kbar = pool_means(k, bk)
    vbar = pool_means(v, bk)
    S, p = router(qbar, kbar, n, bk)
    r_h, k_h = None, None
    price_info = None
    if mode == 0:      # threshold
        t = tiers_threshold(p, cfg_like.tau_hi, cfg_like.tau_lo, cfg_like.top_k,
                            getattr(cfg_like, "tau_skim", 0.0))
    elif mode == 1:    # adaptive
        r_h, k_h, _ = head_retention(p, cfg_like.entropy_samples, cfg_like.keep_min, cfg_like.keep_max)
        t = tiers_adaptive(p, k_h, cfg_like.full_frac, getattr(cfg_like, "tau_skim", 0.0))
    elif mode == 2:    # all full
        t = np.full(p.shape, FULL, dtype=np.uint8)
    elif mode == 4:    # price
        qm, km, vm = block_moments(q, bq), block_moments(k, bk), block_moments(v, bk)
        skim = getattr(cfg_like, "tau_skim", 0.0) > 0
        errs = tile_error_model(qm["m2"], qm["tot_m2"], km["var"], km["tot_m2"], vm["tot_var"],
                                vm["tot_m2"], vm["mnorm"], block_sizes(n, bk), d, skim=skim)
        s2, g, eS, eL = errs[:4]
        eK = errs[4] if skim else None
        pt = corrected_shares(S, g)
        t, objs = tiers_price(pt, eS, eL, cfg_like.price, bk, eK=eK)
        price_info = dict(qm=qm, km=km, vm=vm, s2=s2, g=g, pt=pt, eS=eS, eL=eL, eK=eK, objs=objs)
    else:              # external
        t = np.array(external_tiers, dtype=np.uint8, copy=True)
    t[diagonal_mask(n, bq, bk)] = FULL
    lists, counts = build_lists(t)
    q8, sq, iq = quantise_blocks(q, bq)
    k8, sk, ik = quantise_blocks(k, bk)
    v8, sv, iv = quantise_blocks(v, bk)
    # the MXFP4 copies, where a SKIM tile needs them; the residual-corrected
    # ones where the low tier runs refined
    mx4 = skim_operands(q, k) if np.any(t == SKIM) else None
    refine = refine_operands(q, k) if getattr(cfg_like, "low_refine", 0) else None
    return dict(qbar=qbar, kbar=kbar, vbar=vbar, S=S, p=p, tiers=t, lists=lists, counts=counts,
                q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, r_h=r_h, k_h=k_h, price=price_info, mx4=mx4,
                refine=refine)


def oracle_replan(q, k, v, prev_plan, cfg_like):
    """Plan reuse across diffusion steps (APT: attention probabilities
    predicted across timesteps from their temporal similarity): the previous
    step's tier map is taken as the prediction for this step, and only the
    block means and fp8 codes are recomputed from this step's q, k, v."""
    return oracle_plan(q, k, v, cfg_like, mode=3, external_tiers=prev_plan["tiers"])


def oracle_forward(q, k, v, plan, bq, bk, rows=None, p_codes=None):
    return attention_forward(q, k, v, plan["tiers"], bq, bk, plan["kbar"], plan["vbar"],
                             plan["q8"], plan["sq"], plan["k8"], plan["sk"], plan["v8"], plan["sv"],
                             rows=rows, mx4=plan.get("mx4"), p_codes=p_codes, refine=plan.get("refine"))
