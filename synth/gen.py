"""Seeded, position-correlated Q/K/V generator.

Each token of a (T, Hg, Wg) latent grid gets 8 random Fourier features of its
normalised (t, h, w) position; a seeded Gaussian projection per head maps them
to head_dim channels, and Gaussian noise is added (the workload descriptions'
"8 random Fourier features of the position times a seeded Gaussian projection,
plus noise").  Nearby tokens therefore carry similar keys, which is the
spatio-temporal correlation that makes tile-level routing worthwhile.

Recipe (fixed draw order, one numpy Generator per workload):
  rng = default_rng(SeedSequence([seed, stream]))
  Omega (8x3) ~ N(0, (2*pi*f)^2);  beta (8) ~ U[0, 2*pi)
  per head h: W_Q, W_K (8 x d) ~ N(0, a^2/8), W_V ~ N(0, 1/8) so that V is
              unit-scale; T_h ~ U(0.5, 2) if the
              workload has a temperature; noise E_Q, E_K, E_V ~ N(0, sigma^2)
  phi(n) = sqrt(2) cos(Omega u_n + beta),  u_n = ((t+.5)/T, (h+.5)/Hg, (w+.5)/Wg)
  Q_h = (phi W_Q + E_Q) / T_h,  K_h = phi W_K + E_K,  V_h = phi W_V + E_V
Outputs are [B, H, N, d]; all but the fp32 tiny workload are rounded once to
bf16 (round to nearest even) on the host, and oracle and GPU consume the same
rounded values.

F_CYCLES and A_GAIN were frozen once, on the oracle router at the Wan-like
workload, so that it skips 60-80% of tiles (measured on heads 0, 10, 20, 30:
FULL/LOW/SKIP = 4.6% / 23.5% / 71.9%, every head in [68.5%, 76.2%] skipped);
they are never tuned per run.
"""
import numpy as np

F_CYCLES = 0.5   # spatial frequency scale of the Fourier features (cycles per unit length)
A_GAIN = 3.5     # gain of the per-head Q and K projections


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def positions(grid):
    T, Hg, Wg = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    u = np.stack([(t + 0.5) / T, (h + 0.5) / Hg, (w + 0.5) / Wg], axis=-1)
    return u.reshape(-1, 3)  # token n = (t*Hg + h)*Wg + w


def generate(cfg, seed: int = 0, f_cycles: float = F_CYCLES, a_gain: float = A_GAIN,
             heads=None, noise_sigma=None):
    """Return dict(q, k, v) as float32 arrays [B, H, N, d] holding bf16-exact
    values (fp32 for the tiny workload), plus 'bits' = uint16 bf16 patterns
    (None when the workload is fp32) and the per-head temperatures.

    ``heads`` optionally restricts generation to a subset of head indices; the
    random stream is advanced identically, so head h's tensors do not depend on
    which other heads were requested.
    """
    sid = cfg.seed_stream or cfg.stream
    rng = np.random.default_rng(np.random.SeedSequence([seed, sid]))
    d = cfg.head_dim
    sigma = cfg.noise_sigma if noise_sigma is None else noise_sigma
    omega = rng.normal(0.0, 2.0 * np.pi * f_cycles, size=(8, 3))
    beta = rng.uniform(0.0, 2.0 * np.pi, size=8)
    u = positions(cfg.grid)
    phi = (np.sqrt(2.0) * np.cos(u @ omega.T + beta)).astype(np.float32)  # [N, 8]
    N = u.shape[0]
    want = list(range(cfg.heads)) if heads is None else list(heads)
    B = cfg.batch
    q = np.empty((B, len(want), N, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    temps = np.ones(cfg.heads)
    slot = {h: i for i, h in enumerate(want)}
    for b in range(B):
        for h in range(cfg.heads):
            wq = rng.normal(0.0, a_gain / np.sqrt(8.0), size=(8, d)).astype(np.float32)
            wk = rng.normal(0.0, a_gain / np.sqrt(8.0), size=(8, d)).astype(np.float32)
            wv = rng.normal(0.0, 1.0 / np.sqrt(8.0), size=(8, d)).astype(np.float32)
            th = rng.uniform(0.5, 2.0) if cfg.temperature else 1.0
            temps[h] = th
            if h in slot:
                i = slot[h]
                q[b, i] = (phi @ wq + sigma * rng.standard_normal((N, d), dtype=np.float32)) / np.float32(th)
                k[b, i] = phi @ wk + sigma * rng.standard_normal((N, d), dtype=np.float32)
                v[b, i] = phi @ wv + sigma * rng.standard_normal((N, d), dtype=np.float32)
            else:
                # advance the stream exactly as if the head had been drawn
                rng.standard_normal((3, N, d), dtype=np.float32)
    bits = None
    if not cfg.input_fp32:
        bits = {}
        for name, arr in (("q", q), ("k", k), ("v", v)):
            bb = to_bf16_bits(arr)
            bits[name] = bb
            arr[...] = bf16_bits_to_f32(bb)
    return {"q": q, "k": k, "v": v, "bits": bits, "temps": temps}


def drift_step(g, cfg, step: int, sigma: float, seed: int = 0):
    """The inputs of the next diffusion step: every element of Q, K and V moves
    by independent N(0, sigma^2) noise (a random walk in time, so consecutive
    steps stay similar), then rounds to bf16 again for bf16 workloads.  Drawn
    from SeedSequence([seed, workload, 1000 + step]).  Returns a dict shaped
    like generate()'s."""
    sid = cfg.seed_stream or cfg.stream
    rng = np.random.default_rng(np.random.SeedSequence([seed, sid, 1000 + step]))
    out = {"temps": g["temps"]}
    bits = None if g["bits"] is None else {}
    for name in ("q", "k", "v"):
        x = g[name] + np.float32(sigma) * rng.standard_normal(g[name].shape, dtype=np.float32)
        if bits is not None:
            bits[name] = to_bf16_bits(x)
            x = bf16_bits_to_f32(bits[name])
        out[name] = x.astype(np.float32)
    out["bits"] = bits
    return out
