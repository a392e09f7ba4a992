"""The five workloads on which the three-tier tile-sparse attention is run.

Shapes, tile sizes, thresholds and generator parameters restate the five
workload descriptions that accompany the method: a tiny 4x8x8 latent grid, a
small 8x16x16 grid, a Wan-like 21x30x52 grid with 40 heads, a
HunyuanVideo-like 33x45x80 grid with 24 heads, and the Wan-like grid again with
fine 64x16 tiles and head-adaptive retention.  Token counts come from the
latent grids (frames x height x width).
"""
from dataclasses import dataclass, field, replace
from typing import Tuple

# Mode names follow the C ABI's tattn_mode enumeration.
MODE_THRESHOLD = 0
MODE_ADAPTIVE = 1
MODE_ALL_FULL = 2
MODE_EXTERNAL = 3


@dataclass(frozen=True)
class WorkloadConfig:
    stream: int                 # generator stream id (seeds the random draws)
    name: str
    batch: int
    heads: int
    grid: Tuple[int, int, int]  # latent (T, Hg, Wg); tokens are the row-major flattening
    head_dim: int
    block_q: int
    block_k: int
    tau_hi: float
    tau_lo: float
    mode: int = MODE_THRESHOLD
    top_k: int = 0
    keep_min: float = 0.05
    keep_max: float = 0.50
    full_frac: float = 0.10
    entropy_samples: int = 256
    noise_sigma: float = 0.5
    temperature: bool = False   # per-head temperature T_h ~ U(0.5, 2) divides Q
    input_fp32: bool = False    # the tiny workload is specified in fp32
    seed_stream: int = 0        # draw from another workload's stream (0: own stream)
    tau_skim: float = 0.0       # > 0: the MXFP4 SKIM tier for tau_skim <= p < tau_lo
    extra: dict = field(default_factory=dict)

    @property
    def seq_len(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_qblocks(self) -> int:
        return -(-self.seq_len // self.block_q)

    @property
    def n_kblocks(self) -> int:
        return -(-self.seq_len // self.block_k)

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": WorkloadConfig(1, "tiny", 1, 2, (4, 8, 8), 64, 64, 64, 0.05, 0.005,
                           noise_sigma=0.3, input_fp32=True),
    "small": WorkloadConfig(2, "small", 1, 12, (8, 16, 16), 64, 128, 64, 0.02, 0.002,
                            noise_sigma=0.5),
    "wan_like": WorkloadConfig(3, "wan_like", 1, 40, (21, 30, 52), 128, 128, 64, 0.01, 0.001,
                               noise_sigma=0.5, temperature=True),
    "hunyuan_like": WorkloadConfig(4, "hunyuan_like", 1, 24, (33, 45, 80), 128, 128, 64, 0.01, 0.001,
                                   noise_sigma=0.5, temperature=True),
    "fine_adaptive": WorkloadConfig(5, "fine_adaptive", 1, 40, (21, 30, 52), 128, 64, 16, 0.01, 0.001,
                                    mode=MODE_ADAPTIVE, noise_sigma=0.5, temperature=True, seed_stream=3),
    # finer key granularity than the five described workloads: the same grid
    # and rule with 8-key blocks (4095 key blocks per row)
    "finer_adaptive": WorkloadConfig(6, "finer_adaptive", 1, 40, (21, 30, 52), 128, 64, 8, 0.01, 0.001,
                                     mode=MODE_ADAPTIVE, noise_sigma=0.5, temperature=True, seed_stream=3),
    # the fine workload's grid and 64x16 tiles under threshold tiers with the
    # fourth tier: SKIM steps gather four 16-key blocks
    "fine_skim": WorkloadConfig(10, "fine_skim", 1, 40, (21, 30, 52), 128, 64, 16, 0.01, 0.001,
                                noise_sigma=0.5, temperature=True, seed_stream=3, tau_skim=1e-4),
    # key blocks below 8 keys ("FG-Attn": M x N tiles down to N = 1) on the
    # first frames of the Wan-like grid, sized to the 4096 key blocks a row
    # may hold: 4-key blocks over 10 frames (3900 blocks), one-key blocks over
    # 2 frames (3120 blocks)
    "fg4_adaptive": WorkloadConfig(8, "fg4_adaptive", 1, 40, (10, 30, 52), 128, 64, 4, 0.01, 0.001,
                                   mode=MODE_ADAPTIVE, noise_sigma=0.5, temperature=True, seed_stream=3),
    "fg1_adaptive": WorkloadConfig(9, "fg1_adaptive", 1, 40, (2, 30, 52), 128, 64, 1, 0.01, 0.001,
                                   mode=MODE_ADAPTIVE, noise_sigma=0.5, temperature=True, seed_stream=3),
    # the Wan-like workload with the optional fourth tier: tiles whose router
    # probability lies in [tau_skim, tau_lo) run in MXFP4 instead of being skipped
    "wan_skim": WorkloadConfig(7, "wan_skim", 1, 40, (21, 30, 52), 128, 128, 64, 0.01, 0.001,
                               noise_sigma=0.5, temperature=True, seed_stream=3, tau_skim=2e-4),
}


def get_workload(name: str) -> WorkloadConfig:
    return CONFIGS[name]
