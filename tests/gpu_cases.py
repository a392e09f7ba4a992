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
