"""The C ABI without a GPU: the library loads, exports every function declared
in include/tattn.h, and host-only validation / workspace sizing behave."""
import ctypes
import os
import re

import pytest

import tile_sparse_mixed_amd as tsm
from tile_sparse_mixed_amd import Config, make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tattn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tsm.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def good(**kw):
    base = dict(batch=1, heads=40, seq_len=32760, head_dim=128, block_q=128, block_k=64, tau_hi=0.01, tau_lo=0.001)
    base.update(kw)
    return make_config(**base)


def status(lib, cfg):
    return lib.tattn_validate(ctypes.byref(cfg))


def test_valid_configs(lib):
    assert status(lib, good()) == 0
    assert status(lib, good(head_dim=64, block_q=64, seq_len=256, heads=2)) == 0
    assert status(lib, good(mode="all_full")) == 0
    assert status(lib, good(mode="adaptive")) == 0
    assert status(lib, good(seq_len=118800, heads=24)) == 0
    assert status(lib, good(top_k=10)) == 0
    assert status(lib, good(block_q=64, block_k=8)) == 0                 # 4095 key blocks
    assert status(lib, good(block_q=64, block_k=4, seq_len=16380)) == 0   # 4095 key blocks
    assert status(lib, good(block_q=128, block_k=2, seq_len=8192)) == 0   # 4096 key blocks
    assert status(lib, good(block_q=64, block_k=1, seq_len=4096)) == 0    # one key per block
    assert status(lib, good(mode="price", price=0.01)) == 0
    assert status(lib, good(mode="price", price=0.0)) == 0
    assert status(lib, good(tau_skim=1e-4)) == 0                         # SKIM tier, threshold mode
    assert status(lib, good(tau_skim=0.001)) == 0                        # tau_skim == tau_lo
    assert status(lib, good(mode="external", tau_skim=1e-4)) == 0
    assert status(lib, good(mode="adaptive", block_q=64, block_k=16, tau_skim=1e-4)) == 0   # SKIM below the kept tiles
    # the price router weighs SKIM by its error model: no ordering against tau_lo
    assert status(lib, good(mode="price", price=0.01, tau_skim=0.5)) == 0
    assert status(lib, good(mode="price", price=0.01, tau_skim=-1e-4)) == -1
    assert status(lib, good(mode="price", price=0.01, tau_skim=1e-4, block_q=64, block_k=16)) == 0
    # the SKIM tier on gathered steps, down to one-key blocks
    assert status(lib, good(tau_skim=1e-4, block_q=64, block_k=16)) == 0
    assert status(lib, good(mode="external", tau_skim=1e-4, block_k=8)) == 0
    assert status(lib, good(tau_skim=1e-4, block_q=64, block_k=4, seq_len=16380)) == 0
    assert status(lib, good(mode="external", tau_skim=1e-4, block_k=1, seq_len=4096)) == 0
    # the refined low tier: any block size, not with the SKIM tier, any mode
    for m in ("threshold", "adaptive", "price", "external", "all_full"):
        assert status(lib, good(mode=m, price=0.01, low_refine=True)) == 0, m
    assert status(lib, good(low_refine=True, block_q=64, block_k=16)) == 0
    assert status(lib, good(low_refine=True, block_q=64, block_k=1, seq_len=4096)) == 0
    assert status(lib, good(low_refine=True, tau_skim=1e-4)) == -2
    c = good()
    c.low_refine = 2
    assert status(lib, c) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(heads=-1), -1), (dict(seq_len=0), -1),
    (dict(head_dim=96), -2), (dict(block_q=32), -2), (dict(block_k=32), -2),
    (dict(block_k=16, strides=(40 * 32760 * 128 * 4096, 32760 * 128 * 4096, 128 * 4096)), -2),
    (dict(block_k=8, strides=(40 * 32760 * 128 * 4096, 32760 * 128 * 4096, 128 * 4096)), -2),
    (dict(block_k=8, seq_len=32776), -2),                                # 4097 key blocks
    (dict(block_k=1, seq_len=4097), -2), (dict(block_k=3, seq_len=4096), -2),
    (dict(tau_hi=0.001, tau_lo=0.01), -1), (dict(tau_lo=-0.1), -1), (dict(tau_hi=float("inf")), -1),
    (dict(top_k=-1), -1), (dict(top_k=513), -1), (dict(mode=7), -1),
    (dict(mode="adaptive", keep_min=0.6, keep_max=0.5), -1), (dict(mode="adaptive", full_frac=0.0), -1),
    (dict(mode="adaptive", entropy_samples=0), -1),
    (dict(seq_len=64 * 5000), -2),
    (dict(mode="price", price=-1.0), -1), (dict(mode="price", price=float("nan")), -1),
    (dict(mode=5), -1),
    (dict(tau_skim=-1e-4), -1), (dict(tau_skim=0.002), -1), (dict(tau_skim=float("nan")), -1),
    (dict(tau_skim=1e-4, block_q=64, block_k=2, seq_len=8194), -2),     # 4097 key blocks
])
def test_invalid_configs(lib, kw, code):
    st = status(lib, good(**kw))
    assert st == code, (kw, st, lib.tattn_last_error())
    assert lib.tattn_last_error()


def test_dtype_and_stride_rules(lib):
    c = good()
    c.in_dtype = 1
    assert status(lib, c) == -2
    c = good()
    c.out_dtype = 5
    assert status(lib, c) == -1
    c = good()
    c.stride_n = 100
    assert status(lib, c) == -1
    c = good()
    c.stride_n = 64
    assert status(lib, c) == -1
    assert lib.tattn_validate(None) == -1


def test_workspace_formula(lib):
    c = good()
    n = ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == 0
    BH, Nq, Nk, D = 40, 256, 512, 128
    # dominant regions: E4M3 K and V (1 + 1 B) per key element (FULL tiles read
    # the caller's V, so there is no 16-bit V copy); float64 logits, float32 p,
    # tiers and int16 lists per tile; float32 means and the bf16 hi/lo + fp16
    # pooled operands per block row
    floor = (BH * Nk * 64 * D * 2 + BH * Nq * Nk * (8 + 4 + 1 + 2) + BH * (Nq + 2 * Nk) * D * 4
             + BH * Nk * D * 6)
    assert floor <= n.value <= floor * 1.05
    assert lib.tattn_workspace_bytes(ctypes.byref(good(head_dim=96)), ctypes.byref(n)) == -2
    # the price router adds its second moments and a float64 spread per tile
    m = ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(good(mode="price", price=0.01)), ctypes.byref(m)) == 0
    extra = BH * Nq * Nk * 8 + BH * (Nq + Nk) * D * 4 + BH * (Nq + 4 * Nk) * 4
    assert extra <= m.value - n.value <= extra * 1.05
    # the SKIM tier adds the MXFP4 K codes and scales
    k = ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(good(tau_skim=1e-4)), ctypes.byref(k)) == 0
    extra = BH * Nk * 64 * (D // 2 + D // 32)
    assert extra <= k.value - n.value <= extra * 1.01
    # ... and only where a SKIM tile can occur
    assert lib.tattn_workspace_bytes(ctypes.byref(good(mode="all_full", tau_skim=1e-4)), ctypes.byref(k)) == 0
    assert k.value == n.value
    # the refined low tier adds the MXFP4 K codes and scales and those of its residual
    r = ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(good(low_refine=True)), ctypes.byref(r)) == 0
    extra = 2 * BH * Nk * 64 * (D // 2 + D // 32)
    assert extra <= r.value - n.value <= extra * 1.01
    # the price router with SKIM holds both the moments and the MXFP4 copies
    pk, sk = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(good(mode="price", price=0.01, tau_skim=1e-4)), ctypes.byref(pk)) == 0
    assert lib.tattn_workspace_bytes(ctypes.byref(good(tau_skim=1e-4)), ctypes.byref(sk)) == 0
    assert pk.value - m.value == sk.value - n.value


def test_plan_rejects_bad_pointers_before_any_launch(lib):
    c = good(seq_len=256, heads=2, head_dim=64, block_q=64)
    out = ctypes.c_void_p()
    assert lib.tattn_plan(ctypes.byref(c), None, None, None, None, 0, None, ctypes.byref(out)) == -1
    # misaligned q (not 16-byte) is rejected on the host
    assert lib.tattn_plan(ctypes.byref(c), 8, 16, 32, 256, 1 << 30, None, ctypes.byref(out)) == -1
    # workspace too small / misaligned / missing
    assert lib.tattn_plan(ctypes.byref(c), 16, 32, 48, 256, 16, None, ctypes.byref(out)) == -3
    assert lib.tattn_plan(ctypes.byref(c), 16, 32, 48, 300, 1 << 30, None, ctypes.byref(out)) == -3
    assert lib.tattn_plan(ctypes.byref(c), 16, 32, 48, None, 1 << 30, None, ctypes.byref(out)) == -3
    assert out.value is None
    assert lib.tattn_forward(None, 16, 32, 48, 64, None) == -1
    assert lib.tattn_plan_stats(None, None) == -1
    assert lib.tattn_plan_get_mx4(None, None, None, None, None) == -1
    lib.tattn_plan_destroy(None)


def test_config_layout_matches_header(lib):
    """The binding's struct has the header's field order; low_refine is last."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} tattn_config;", text, flags=re.S).group(1)
    names = re.findall(r"([a-z_]+)\s*[,;]", body)
    assert names == [f for f, _ in Config._fields_]
    assert ctypes.sizeof(Config) == 104


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.tattn_status_str(s)
    assert lib.tattn_status_str(-99) == b"unknown status"


def test_forward_dump_rejects_bad_arguments(lib):
    """Argument checks of the code-dump forward run before any device call."""
    buf = (ctypes.c_uint8 * 64)()
    slot = (ctypes.c_int32 * 4)()
    assert lib.tattn_forward_dump(None, None, None, None, None, None, 1, ctypes.addressof(buf), None) == -1
    assert lib.tattn_forward_dump(None, None, None, None, None, ctypes.addressof(slot), 0,
                                  ctypes.addressof(buf), None) == -1
    assert lib.tattn_forward_dump(None, None, None, None, None, ctypes.addressof(slot), 1,
                                  ctypes.addressof(buf) + 1, None) == -1


@pytest.mark.parametrize("mode,extra", [("adaptive", {}), ("adaptive", dict(keep_min=0.5, keep_max=0.5)),
                                        ("adaptive", dict(tau_skim=3e-4)),
                                        ("threshold", dict(top_k=3)), ("threshold", dict(top_k=1)),
                                        ("threshold", dict(top_k=3, tau_skim=3e-4)),
                                        ("threshold", {}), ("price", dict(price=0.01))])
@pytest.mark.parametrize("tiles", [(128, 64), (64, 64), (64, 16), (64, 8), (128, 16)])
def test_list_bound_holds_every_row(mode, extra, tiles):
    """The fused kernel's per-row list bound (host only) against the most kept
    tiles any row of the oracle's plan holds, on small generated workloads."""
    import numpy as np
    from oracle import tattn as T
    from synth import CONFIGS, generate
    bq, bk = tiles
    cfg = CONFIGS["small"].with_(heads=2, grid=(4, 9, 13), block_q=bq, block_k=bk,
                                 mode={"threshold": 0, "adaptive": 1, "price": 4}[mode],
                                 **{k: v for k, v in extra.items() if k != "price"})
    c = make_config(1, cfg.heads, cfg.seq_len, cfg.head_dim, bq, bk, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo,
                    top_k=cfg.top_k, mode=mode, keep_min=cfg.keep_min, keep_max=cfg.keep_max,
                    full_frac=cfg.full_frac, price=extra.get("price", 0.0), tau_skim=extra.get("tau_skim", 0.0))
    bound = tsm.list_bound(c)
    assert 1 <= bound <= cfg.n_kblocks
    g = generate(cfg)

    class OC:
        block_q, block_k, tau_hi, tau_lo = bq, bk, float(np.float32(cfg.tau_hi)), float(np.float32(cfg.tau_lo))
        top_k, keep_min, keep_max, full_frac = cfg.top_k, float(np.float32(cfg.keep_min)), \
            float(np.float32(cfg.keep_max)), float(np.float32(cfg.full_frac))
        entropy_samples, price = cfg.entropy_samples, float(np.float32(extra.get("price", 0.0)))
        tau_skim = float(np.float32(extra.get("tau_skim", 0.0)))
        mode = cfg.mode
    for h in range(cfg.heads):
        o = T.oracle_plan(g["q"][0, h], g["k"][0, h], g["v"][0, h], OC)
        assert int((o["tiers"] != T.SKIP).sum(axis=1).max()) <= bound, (mode, tiles, h)
