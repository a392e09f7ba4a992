"""CPU oracle for three-tier tile-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's cpu_baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it.

Plain numpy, float64 unless a step's decision is taken in the kernel's
precision (the fp8 codes are decided on float32 values, as the kernel does).
Each function names the passage of the pages it follows:
  * "Triage" abstract (zhuanzhiai page): skip a tile by replacing it with its
    block means; three tiers; one fused pass.
  * "APT" abstract (Lattice page): attention probability as the importance
    metric; dual thresholds select elements and assign precision.
  * "HierPAS" abstract (conference page): lightweight eager estimate of the
    attention pattern; sampling-based entropy gives head-wise retention
    ratios; progressively lower precision for less critical regions; top-k.
  * "FG-Attn" abstract (searcharxiv author page): M x N tile granularity.
  * "Triage" abstract again for the optional fourth tier: skimming a tile in a
    4-bit format (here OCP MXFP4, oracle/mxfp4.py).
Formulas the pages leave open follow the readings listed with the design
(block-mean router with +ln n_J; the low tier quantises Q, K, V to E4M3 with
one scale per block and its probabilities to E4M3 against the tile-local row
maximum times 448, and sums those quantised probabilities into the row
normaliser).

Parity status: every function is pinned by tests/test_oracle_*.py except the
entropy -> retention-ratio mapping of the head-adaptive mode, whose formula the
pages do not fix ("parity unpinned"; only its [5%, 50%] clip is external), and
the price router's error model as a predictor (its exact identities and its
derivation are pinned, its accuracy as a predictor is not: "parity unpinned").
"""
from . import e4m3, mxfp4  # noqa: F401
from .tattn import (  # noqa: F401
    SKIP, LOW, FULL, SKIM, skim_operands, refine_operands, refine_scores, block_sizes, pool_means, router, tiers_threshold, tiers_adaptive,
    head_retention, diagonal_mask, build_lists, quantise_blocks, dequantise, quantised_probabilities, low_scores,
    attention_forward,
    oracle_plan, oracle_forward, naive_attention, effective_weights,
)
