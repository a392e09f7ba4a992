"""P4: the oracle's router, tier map, top-k and lists against brute force on
tiny inputs: scalar triple loops with math.fsum for the means and
probabilities, direct comparisons for the thresholds, exhaustive subset search
for top-k, and an interval test for the diagonal."""
import itertools
import math

import numpy as np
import pytest

from oracle import tattn as T
from oracle.tattn import FULL, LOW, SKIP


def brute_p(q, k, bq, bk):
    n, d = q.shape
    nq, nk = -(-n // bq), -(-n // bk)
    qb = [[math.fsum(float(q[i, c]) for i in range(I * bq, min(n, (I + 1) * bq))) /
           (min(n, (I + 1) * bq) - I * bq) for c in range(d)] for I in range(nq)]
    kb = [[math.fsum(float(k[j, c]) for j in range(J * bk, min(n, (J + 1) * bk))) /
           (min(n, (J + 1) * bk) - J * bk) for c in range(d)] for J in range(nk)]
    qb = [[float(np.float32(x)) for x in row] for row in qb]    # means are stored as float32
    kb = [[float(np.float32(x)) for x in row] for row in kb]
    P = []
    for I in range(nq):
        logits = []
        for J in range(nk):
            nJ = min(n, (J + 1) * bk) - J * bk
            logits.append(math.fsum(qb[I][c] * kb[J][c] for c in range(d)) / math.sqrt(d) + math.log(nJ))
        mx = max(logits)
        ex = [math.exp(x - mx) for x in logits]
        z = math.fsum(ex)
        P.append([x / z for x in ex])
    return np.array(P)


def brute_tiers(P, n, bq, bk, tau_hi, tau_lo, top_k):
    nq, nk = P.shape
    t = np.zeros((nq, nk), np.uint8)
    for I in range(nq):
        keep = set(range(nk))
        if top_k > 0:
            best, best_key = None, None
            for sub in itertools.combinations(range(nk), min(top_k, nk)):
                key = (-math.fsum(P[I, j] for j in sub), sub)     # max mass, then lexicographically smallest
                if best_key is None or key < best_key:
                    best, best_key = sub, key
            keep = set(best)
        for J in range(nk):
            if J not in keep:
                t[I, J] = SKIP
            elif P[I, J] >= tau_hi:
                t[I, J] = FULL
            elif P[I, J] >= tau_lo:
                t[I, J] = LOW
            else:
                t[I, J] = SKIP
            lo_q, hi_q = I * bq, min(n, (I + 1) * bq) - 1
            lo_k, hi_k = J * bk, min(n, (J + 1) * bk) - 1
            if not (hi_k < lo_q or lo_k > hi_q):
                t[I, J] = FULL
    return t


CASES = [(40, 4, 8, 8, 0), (64, 6, 16, 8, 3), (100, 5, 32, 16, 2), (77, 8, 16, 12, 4), (500, 4, 128, 64, 5),
         (512, 3, 64, 64, 0), (45, 4, 7, 9, 3)]


@pytest.mark.parametrize("n,d,bq,bk,top_k", CASES)
def test_bruteforce_router_and_tiers(n, d, bq, bk, top_k):
    r = np.random.default_rng(n * 31 + d)
    q = (r.standard_normal((n, d)) * 2).astype(np.float32)
    k = (r.standard_normal((n, d)) * 2).astype(np.float32)
    qbar, kbar = T.pool_means(q, bq), T.pool_means(k, bk)
    _, p = T.router(qbar, kbar, n, bk)
    P = brute_p(q, k, bq, bk)
    assert np.max(np.abs(p - P) / P) < 1e-12
    tau_hi, tau_lo = float(np.quantile(P, 0.75)), float(np.quantile(P, 0.35))
    t = T.tiers_threshold(p, tau_hi, tau_lo, top_k)
    t[T.diagonal_mask(n, bq, bk)] = FULL
    tb = brute_tiers(P, n, bq, bk, tau_hi, tau_lo, top_k)
    band = (np.abs(P - tau_hi) <= 1e-9 * tau_hi) | (np.abs(P - tau_lo) <= 1e-9 * tau_lo)
    assert np.array_equal(t[~band], tb[~band])


def test_bruteforce_topk_ties_go_to_lower_index():
    p = np.array([[0.2, 0.1, 0.2, 0.2, 0.3]])
    t = T.tiers_threshold(p, 0.0, 0.0, top_k=3)
    assert t.tolist() == [[FULL, SKIP, FULL, SKIP, FULL]]


@pytest.mark.parametrize("nk,k_h,frac", [(8, 5, 0.1), (7, 7, 0.5), (9, 2, 0.1), (6, 6, 0.34)])
def test_bruteforce_adaptive_rank_tiers(nk, k_h, frac):
    r = np.random.default_rng(nk * 10 + k_h)
    p = r.dirichlet(np.ones(nk), size=5)
    t = T.tiers_adaptive(p, k_h, frac)
    nfull = math.ceil(frac * k_h)
    for I in range(5):
        for J in range(nk):
            # rank = number of tiles strictly ahead in (p desc, J asc) order
            rank = sum(1 for J2 in range(nk) if p[I, J2] > p[I, J] or (p[I, J2] == p[I, J] and J2 < J))
            want = FULL if rank < nfull else (LOW if rank < k_h else SKIP)
            assert t[I, J] == want


@pytest.mark.parametrize("nk,k_h,frac,tau", [(8, 3, 0.1, 0.08), (9, 2, 0.5, 0.02), (6, 6, 0.34, 0.1)])
def test_bruteforce_adaptive_rank_tiers_with_skim(nk, k_h, frac, tau):
    """With the fourth tier, the tiles outside the top k_h split at tau_skim:
    SKIM at or above it, SKIP below; the kept tiles are as without it."""
    from oracle import SKIM
    r = np.random.default_rng(nk * 100 + k_h)
    p = r.dirichlet(np.ones(nk), size=5)
    t = T.tiers_adaptive(p, k_h, frac, tau_skim=tau)
    t0 = T.tiers_adaptive(p, k_h, frac)
    nfull = math.ceil(frac * k_h)
    tau32 = float(np.float32(tau))
    for I in range(5):
        for J in range(nk):
            rank = sum(1 for J2 in range(nk) if p[I, J2] > p[I, J] or (p[I, J2] == p[I, J] and J2 < J))
            want = FULL if rank < nfull else (LOW if rank < k_h else (SKIM if p[I, J] >= tau32 else SKIP))
            assert t[I, J] == want
    assert np.array_equal(t[t0 != SKIP], t0[t0 != SKIP])
    assert np.array_equal(T.tiers_adaptive(p, k_h, frac, tau_skim=0.0), t0)


def test_head_retention_clip_and_ceiling():
    nk = 100
    uniform = np.full((8, nk), 1.0 / nk)            # entropy ln(nk): perplexity nk -> clipped to 0.5
    r, k, _ = T.head_retention(uniform, 256, 0.05, 0.5)
    assert r == 0.5 and k == 50
    peaked = np.zeros((8, nk))
    peaked[:, 0] = 1.0                               # entropy 0: perplexity 1 -> 1/nk -> clipped to 0.05
    r, k, _ = T.head_retention(peaked, 256, 0.05, 0.5)
    assert r == 0.05 and k == 5
    two = np.zeros((8, nk))
    two[:, :20] = 1.0 / 20                          # perplexity exactly 20 -> r = 0.2, k = 20
    r, k, _ = T.head_retention(two, 256, 0.05, 0.5)
    assert abs(r - 0.2) < 1e-12 and k in (20, 21)


def test_sampled_rows_stride():
    # 512 query blocks, 256 samples -> every other block starting at 0
    p = np.zeros((512, 4))
    p[:, 0] = 1.0
    p[1::2] = 0.25                                   # odd rows are uniform: they must not be sampled
    r, k, H = T.head_retention(p, 256, 0.0, 1.0)
    assert H.shape == (256,) and np.all(H == 0)
