"""Pins of the oracle at key blocks below 8 keys ("FG-Attn": M x N tiles
down to N = 1), against closed forms that hold only there.

- One-key blocks, every tile SKIP but the diagonal: a block's pooled key and
  value are the key and value themselves and ln n_J = 0, so the output is
  dense softmax attention.
- One-key blocks, every tile LOW but the diagonal: a block's probabilities
  are quantised against its own maximum, which is its only score, so every
  code is 448 and the low tier reduces to e^{s^_j} weights on the E4M3
  scores with the dequantised values.
- Every tile FULL at 1-, 2- and 4-key blocks is dense attention.
"""
import math
from types import SimpleNamespace

import numpy as np

from oracle import FULL, LOW, SKIP, e4m3
from oracle import tattn as T


def _cfg(bq, bk):
    return SimpleNamespace(block_q=bq, block_k=bk, tau_hi=0.05, tau_lo=0.005, top_k=0, mode=3,
                           keep_min=0.05, keep_max=0.5, full_frac=0.1, entropy_samples=256)


def _qkv(n, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)).astype(np.float32) for _ in range(3)]


def _dense(q, k, v):
    """softmax(q k^T / sqrt(d)) v in float64, written out."""
    s = q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(q.shape[1])
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ v.astype(np.float64)) / w.sum(axis=1, keepdims=True)


def _forward(q, k, v, c, fill):
    n = q.shape[0]
    nq, nk = -(-n // c.block_q), -(-n // c.block_k)
    plan = T.oracle_plan(q, k, v, c, mode=3, external_tiers=np.full((nq, nk), fill, np.uint8))
    out = T.attention_forward(q, k, v, plan["tiers"], c.block_q, c.block_k, plan["kbar"], plan["vbar"],
                              plan["q8"], plan["sq"], plan["k8"], plan["sk"], plan["v8"], plan["sv"])
    return out, plan


def test_one_key_skip_blocks_are_dense_attention():
    q, k, v = _qkv(150, 32, 1)                       # ragged last query block
    out, plan = _forward(q, k, v, _cfg(64, 1), SKIP)
    assert np.any(plan["tiers"] == SKIP) and np.any(plan["tiers"] == FULL)
    assert np.abs(out - _dense(q, k, v)).max() < 1e-12


def test_one_key_low_blocks_drop_the_probability_quantisation():
    n, d, bq = 130, 64, 64
    q, k, v = _qkv(n, d, 2)
    out, plan = _forward(q, k, v, _cfg(bq, 1), LOW)
    t = plan["tiers"]
    qd = e4m3.decode(plan["q8"]).astype(np.float64)             # [n, d] code values
    kd = e4m3.decode(plan["k8"]).astype(np.float64)
    vd = e4m3.decode(plan["v8"]).astype(np.float64)
    sq = np.repeat(plan["sq"].astype(np.float64), bq)[:n]        # per query row
    sk = plan["sk"].astype(np.float64)                           # per key (one-key blocks)
    vhat = (vd * plan["sv"].astype(np.float32)[:, None]).astype(np.float32).astype(np.float64)
    want = np.zeros((n, d))
    for i in range(n):
        I = i // bq
        s_low = (qd[i] @ kd.T) * sq[i] * sk / math.sqrt(d)
        s_full = (q[i].astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
        full = t[I] == FULL
        s = np.where(full, s_full, s_low)
        vals = np.where(full[:, None], v.astype(np.float64), vhat)
        w = np.exp(s - s.max())
        want[i] = w @ vals / w.sum()
    assert np.abs(out - want).max() < 1e-12


def test_all_full_at_small_blocks_is_dense_attention():
    q, k, v = _qkv(100, 32, 3)
    ref = _dense(q, k, v)
    for bk in (1, 2, 4):
        out, _ = _forward(q, k, v, _cfg(64, bk), FULL)
        assert np.abs(out - ref).max() < 1e-12, bk
