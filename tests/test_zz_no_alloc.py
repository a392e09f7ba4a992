"""The entry point that allocates nothing (tattn_attention_static): plan and
forward with the library's static device workspace, against tattn_plan +
tattn_forward on the same inputs, on two calls in a row (the second on a
smaller problem, so the static array still holds the first call's contents),
and the size limit."""
import ctypes

import numpy as np
import pytest

from synth import CONFIGS

from gpu_cases import device_inputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _both(tsm, dev, cfg, out_fp32):
    kw = dict(block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo, out_fp32=out_fp32)
    p = tsm.plan(dev["q"], dev["k"], dev["v"], **kw)
    ref = tsm.forward(p, dev["q"], dev["k"], dev["v"])
    got = tsm.attention_static(dev["q"], dev["k"], dev["v"], **kw)
    return ref.float().cpu().numpy(), got.float().cpu().numpy()


def test_static_workspace_matches_plan_and_forward():
    import torch
    import tile_sparse_mixed_amd as tsm
    cases = [("one Wan-like head, 32760 x d128, 128x64 tiles", CONFIGS["wan_like"].with_(heads=1), False),
             ("small, 2048 x 12 heads x d64", CONFIGS["small"], True)]
    for what, cfg, out_fp32 in cases:
        _log(f"[static] {what}")
        g, dev = device_inputs(cfg)
        ref, got = _both(tsm, dev, cfg, out_fp32)
        torch.cuda.synchronize()
        err = np.abs(got.astype(np.float64) - ref)
        _log(f"  vs plan + forward: max-abs {err.max():.3e}, bit-identical {np.array_equal(got, ref)}")
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, (what, err.max(), err.mean())
        assert np.array_equal(got, ref), what        # the same kernels on the same inputs


def test_static_workspace_limit_and_mode():
    import tile_sparse_mixed_amd as tsm
    lib = tsm.load_library()
    big = tsm.make_config(1, 8, 32760, 128, 128, 64, tau_hi=0.01, tau_lo=0.001)      # ~87 MiB of workspace
    need = ctypes.c_size_t()
    assert lib.tattn_workspace_bytes(ctypes.byref(big), ctypes.byref(need)) == 0
    # the fake pointers below are only safe while the call must refuse the size
    assert need.value > (64 << 20), need.value
    fake = ctypes.c_void_p(1 << 20)                                                  # aligned, never dereferenced
    assert lib.tattn_attention_static(ctypes.byref(big), fake, fake, fake, fake, None) == -3
    assert b"static scratch" in lib.tattn_last_error()
    ext = tsm.make_config(1, 1, 256, 64, 64, 64, mode="external")
    assert lib.tattn_attention_static(ctypes.byref(ext), fake, fake, fake, fake, None) == -5
