"""Benchmark of the three-tier tile-sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: plan
(block pooling + fp8 quantisation, router + tiers + lists) then the fused
three-tier forward.  Workload: the Wan-like 21x30x52 grid (32760 tokens), 40
heads, d = 128, 128x64 tiles, tau_hi = 0.01, tau_lo = 0.001, bf16 inputs
already resident in HBM.

Prints ONE JSON line.  `value` is dense-equivalent TFLOP/s of the step
(4 N^2 d H / t_step).  The roofline entry covers the fused kernel (K3): the
MFMA utilisation on kept tiles, U = (F_bf16 / P_bf16 + F_fp8 / P_fp8 + F_fp4 /
P_fp4) / t, with F the algorithmic flops of the tier map (FULL tiles 4 m n d in
bf16, LOW tiles 4 m n d in fp8, SKIM tiles 2 m n d in fp4 plus 2 m n d in fp8,
SKIP tiles 4 m d in bf16) and t the kernel's average launch time measured with
HIP events on the stream it runs on; reported as bf16-equivalent TFLOP/s
against the 2.5 PFLOP/s dense bf16 peak, so frac = U.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16 MFMA
PEAK_FP8 = 5000.0    # TFLOP/s, MI355X dense fp8 MFMA
PEAK_FP4 = 10100.0   # TFLOP/s, MI355X dense fp4 MFMA
PEAK_HBM = 8000.0    # GB/s
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k3_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan_like",
                    choices=["tiny", "small", "wan_like", "hunyuan_like", "fine_adaptive", "finer_adaptive",
                             "wan_skim", "fine_skim", "fg4_adaptive", "fg1_adaptive"])
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-allfull", action="store_true", help="skip the all-full comparison")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--gen-heads", type=int, default=0,
                    help="generate only this many heads and tile them to the workload's head count (same shapes "
                         "and launch; for the large workloads, whose full host-side generation takes minutes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for counter scaling)")
    ap.add_argument("--low-refine", action="store_true",
                    help="score LOW tiles on MXFP4 with residual correction instead of E4M3 (and compare)")
    ap.add_argument("--price", type=float, default=None,
                    help="route with the price router at this price instead of the workload's own tier rule")
    return ap.parse_args()


def source_hash():
    """Hash of the fused kernel's code (comments and blank lines stripped, so
    an edit of a comment does not void the recorded counters)."""
    h = hashlib.sha256()
    for f in ("k3_attn.hpp", "k3_attn.hip", "k3_bk64.hip", "tattn_device.hpp"):
        with open(os.path.join(ROOT, "tile_sparse_mixed_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        code = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in code if ln.strip()).encode())
    return h.hexdigest()[:16]


def load_counters(workload):
    """Counter figures of one K3 launch from committed rocprofv3 runs (HBM bytes
    from FETCH_SIZE / WRITE_SIZE, copy-calibrated; the MFMA-busy fraction), if
    they were taken on the current kernel source and this workload; else {}."""
    try:
        with open(COUNTERS_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return {}
    if t.get("source_hash") != source_hash() or t.get("workload") != workload:
        return {}
    return t


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_vendor():
    """The BLAS library numpy was built against, as numpy reports it."""
    import numpy as np
    try:
        info = np.show_config(mode="dicts")
        blas = info.get("Build Dependencies", {}).get("blas", {})
        return f"{blas.get('name', 'unknown')} {blas.get('version', '')}".strip()
    except Exception:   # older numpy without mode="dicts"
        return "unknown"


def _oracle_worker(args):
    """One pool worker: the oracle's plan of one head (timed), then forward
    query blocks in a fixed random order until the budget is spent (timed)."""
    q, k, v, ocfg, n_qblocks, block_q, block_k, budget_s, seed = args
    from threadpoolctl import threadpool_limits
    import numpy as np
    from oracle import tattn as T
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        plan = T.oracle_plan(q, k, v, ocfg)
        t_plan = time.perf_counter() - t0
        rows = blocks = 0
        t1 = time.perf_counter()
        for I in np.random.default_rng(seed).permutation(n_qblocks):
            T.oracle_forward(q, k, v, plan, block_q, block_k, rows=[int(I)])
            rows += min(block_q, q.shape[0] - int(I) * block_q)
            blocks += 1
            if time.perf_counter() - t1 > budget_s:
                break
        t_fwd = time.perf_counter() - t1
    return t_plan, t_fwd, rows, blocks


class _OracleCfg:
    """The oracle's view of a workload's tier rule (plain attributes, picklable)."""

    def __init__(self, cfg, price):
        import numpy as np
        f32 = lambda x: float(np.float32(x))
        self.block_q, self.block_k = cfg.block_q, cfg.block_k
        self.tau_hi, self.tau_lo, self.tau_skim = f32(cfg.tau_hi), f32(cfg.tau_lo), f32(cfg.tau_skim)
        self.top_k, self.mode = cfg.top_k, (4 if price is not None else cfg.mode)
        self.keep_min, self.keep_max, self.full_frac = f32(cfg.keep_min), f32(cfg.keep_max), f32(cfg.full_frac)
        self.entropy_samples = cfg.entropy_samples
        self.price = f32(price) if price is not None else 0.0


def cpu_baseline(g, cfg, budget_s, price=None):
    """The oracle on the host's cores: a process pool over heads, one BLAS
    thread per worker, each worker owning one head: its full plan (pool,
    router, tiers) timed, then query blocks of its forward until the budget is
    spent.  Returns the pool's aggregate dense-equivalent TFLOP/s (each
    worker's rows at 4 rows N d, its plan charged pro rata to the query blocks
    it ran), with plan and forward times reported separately."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    workers = max(1, min(16, len(os.sched_getaffinity(0)), g["q"].shape[1]))
    oc = _OracleCfg(cfg, price)
    jobs = [(g["q"][0, h], g["k"][0, h], g["v"][0, h], oc, cfg.n_qblocks, cfg.block_q, cfg.block_k, budget_s, h)
            for h in range(workers)]
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_worker, jobs))
    wall = time.perf_counter() - t0
    N, d = g["q"].shape[2], g["q"].shape[3]
    rate = 0.0
    for t_plan, t_fwd, rows, blocks in res:
        rate += 4.0 * rows * N * d / (t_fwd + t_plan * blocks / cfg.n_qblocks)
    t_plan = sum(r[0] for r in res) / len(res)
    t_blk = sum(r[1] for r in res) / sum(r[3] for r in res)
    return {"value": round(rate / 1e12, 5), "unit": "TFLOP/s (dense-equivalent)", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(), "blas": _blas_vendor(),
            "plan_s_per_head": round(t_plan, 3), "forward_s_per_query_block": round(t_blk, 4),
            "step_s_estimate": round((t_plan + t_blk * cfg.n_qblocks) * cfg.heads / workers, 1),
            "sample": f"{workers} worker processes (one BLAS thread each), one head each of {cfg.heads}: the full "
                      f"plan ({t_plan:.2f} s per head) then {sum(r[3] for r in res)} query blocks of forward in "
                      f"total ({t_blk:.3f} s each); numpy float64 oracle, pool wall {wall:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads would shard across GPUs with no exchange; that path is not implemented)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import tile_sparse_mixed_amd as tsm
    from synth import CONFIGS, generate

    cfg = CONFIGS[args.workload]
    if cfg.mode not in (0, 1):
        print("bench.py: only threshold and entropy-adaptive workloads are benchmarked", file=sys.stderr)
        sys.exit(2)
    run_mode = "price" if args.price is not None else ("adaptive" if cfg.mode == 1 else "threshold")
    print(f"[bench] generating {cfg.name}: N={cfg.seq_len} H={cfg.heads} d={cfg.head_dim}", file=sys.stderr,
          flush=True)
    tiled = 0 < args.gen_heads < cfg.heads
    g = generate(cfg.with_(heads=args.gen_heads) if tiled else cfg)
    dev = {}
    for n in ("q", "k", "v"):
        t = torch.from_numpy(g["bits"][n].view(np.int16)).view(torch.bfloat16).cuda()
        if tiled:
            t = t.index_select(1, torch.arange(cfg.heads, device="cuda") % args.gen_heads).contiguous()
        dev[n] = t
    q, k, v = dev["q"], dev["k"], dev["v"]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def mk(mode, ws=None, skim=True, refine=None):
        refine = args.low_refine if refine is None else refine
        return tsm.plan(q, k, v, block_q=cfg.block_q, block_k=cfg.block_k, tau_hi=cfg.tau_hi, tau_lo=cfg.tau_lo,
                        top_k=cfg.top_k, mode=mode, keep_min=cfg.keep_min, keep_max=cfg.keep_max,
                        full_frac=cfg.full_frac, entropy_samples=cfg.entropy_samples, workspace=ws,
                        price=args.price or 0.0, tau_skim=cfg.tau_skim if mode != "all_full" and skim else 0.0,
                        low_refine=refine and mode != "all_full")

    out = torch.empty_like(q)
    plan = mk(run_mode)
    tsm.forward(plan, q, k, v, out)
    torch.cuda.synchronize()
    st = plan.stats()
    # tiles whose router probability lies within 1e-5 (relative) of a threshold:
    # the band where a tier may legitimately differ between implementations
    n_band = None
    if run_mode == "threshold":
        pr = plan.tiers(with_p=True)[1]
        n_band = int(sum(np.count_nonzero(np.abs(pr - np.float32(t)) <= 1e-5 * np.float32(t))
                         for t in (cfg.tau_hi, cfg.tau_lo) + ((cfg.tau_skim,) if cfg.tau_skim > 0 else ())))
        del pr
    kh_summary = None
    if run_mode == "adaptive":   # k_h per head: min / median / max and a 10-bin histogram
        kh = plan.kh()[0]
        hist, edges = np.histogram(kh, bins=10)
        kh_summary = {"k_h_min": int(kh.min()), "k_h_median": float(np.median(kh)), "k_h_max": int(kh.max()),
                      "of_n_kblocks": cfg.n_kblocks, "histogram": hist.tolist(),
                      "bin_edges": [round(float(e), 1) for e in edges]}

    ws = torch.empty_like(plan.workspace)   # the timed steps re-plan into one workspace

    def step():
        p = mk(run_mode, ws)
        tsm.forward(p, q, k, v, out)
        return p

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-stage times on the same stream: plan alone, forward alone.  One event
    # per repetition, no synchronisation in between: mean, median and min.
    def timed(fn, reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        return ev[0].elapsed_time(ev[-1]) / reps, per[len(per) // 2], per[0]

    ms_plan, med_plan, min_plan = timed(lambda: mk(run_mode, ws), args.steps)
    ms_k3, med_k3, min_k3 = timed(lambda: tsm.forward(plan, q, k, v, out), args.steps)
    # plan reuse across diffusion steps: re-pool and re-quantise (K1) only
    ms_replan = timed(lambda: tsm.replan(plan, q, k, v), args.steps)[0]
    ms_reuse = timed(lambda: (tsm.replan(plan, q, k, v), tsm.forward(plan, q, k, v, out)), args.steps)[0]

    ms_allfull = None
    quality = None
    skim_cmp = None
    refine_cmp = None
    if not args.no_allfull:
        pf = mk("all_full")
        dense_out = torch.empty_like(out)
        tsm.forward(pf, q, k, v, dense_out)
        ms_allfull = timed(lambda: tsm.forward(pf, q, k, v, dense_out), max(3, args.steps // 4))[0]
        del pf
        # approximation quality of the sparse output against the all-full one
        # (reported, not gated: the pages give no bound)
        a, b = out.float(), dense_out.float()
        diff = (a - b).flatten(2)
        num = diff.pow(2).sum(-1)
        quality = {"vs": "all-full forward (bf16 output)",
                   "max_abs": round(float(diff.abs().max()), 5),
                   "rel_l2": round(float((num.sum() / b.flatten(2).pow(2).sum()).sqrt()), 6),
                   "cosine_min_row": round(float(torch.nn.functional.cosine_similarity(a, b, dim=-1).min()), 6)}
        if cfg.tau_skim > 0 and run_mode == "threshold":
            # the SKIM band run as LOW tiles and as SKIP tiles (same map otherwise):
            # what the fourth tier costs and buys against its neighbours
            t_map = plan.tiers()
            skim_cmp = {"skim_share": round(float((t_map == tsm.SKIM).mean()), 4),
                        "with_skim": {"forward_ms": round(ms_k3, 4), "rel_l2": quality["rel_l2"]}}
            for name, tier in (("band_as_low", tsm.LOW), ("band_as_skip", tsm.SKIP)):
                pe = mk("external", skim=False)   # no SKIM bytes: the kernel without the tier
                pe.set_tiers(np.where(t_map == tsm.SKIM, tier, t_map).astype(np.uint8))
                alt = torch.empty_like(out)
                tsm.forward(pe, q, k, v, alt)
                ms_alt = timed(lambda: tsm.forward(pe, q, k, v, alt), args.steps)[0]
                af = alt.float()
                rel = float(((af - b).flatten(2).pow(2).sum() / b.flatten(2).pow(2).sum()).sqrt())
                skim_cmp[name] = {"forward_ms": round(ms_alt, 4), "rel_l2": round(rel, 6)}
                del pe, alt, af
        if args.low_refine:
            # the same tier map with LOW tiles scored on the E4M3 copies: what
            # the residual-corrected MXFP4 scores cost and buy against them
            refine_cmp = {"low_share": round(float((plan.tiers() == tsm.LOW).mean()), 4),
                          "refined_mxfp4": {"forward_ms": round(ms_k3, 4), "rel_l2": quality["rel_l2"]}}
            pe = mk(run_mode, refine=False)
            alt = torch.empty_like(out)
            tsm.forward(pe, q, k, v, alt)
            ms_alt = timed(lambda: tsm.forward(pe, q, k, v, alt), args.steps)[0]
            af = alt.float()
            rel = float(((af - b).flatten(2).pow(2).sum() / b.flatten(2).pow(2).sum()).sqrt())
            refine_cmp["e4m3"] = {"forward_ms": round(ms_alt, 4), "rel_l2": round(rel, 6)}
            # each low tier's own error: against the same map with its LOW
            # tiles run as FULL tiles (bf16 scores, exact probabilities)
            pf = mk("external", refine=False)
            t_map = plan.tiers()
            pf.set_tiers(np.where(t_map == tsm.LOW, tsm.FULL, t_map).astype(np.uint8))
            ref = torch.empty_like(out)
            tsm.forward(pf, q, k, v, ref)
            rf = ref.float()
            den = rf.flatten(2).pow(2).sum()
            for key, o_ in (("refined_mxfp4", a), ("e4m3", af)):
                refine_cmp[key]["rel_l2_vs_low_as_full"] = round(float(((o_ - rf).flatten(2).pow(2).sum() / den).sqrt()), 6)
            refine_cmp["rel_l2_refined_vs_e4m3"] = round(float(((a - af).flatten(2).pow(2).sum() / den).sqrt()), 6)
            del pe, alt, af, pf, ref, rf
        del dense_out, a, b, diff, num

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    dense = st["flops_dense"]
    executed = st["flops_bf16"] + st["flops_fp8"] + st["flops_fp4"]
    bf16_equiv = st["flops_bf16"] + st["flops_fp8"] * PEAK_BF16 / PEAK_FP8 + st["flops_fp4"] * PEAK_BF16 / PEAK_FP4
    achieved = bf16_equiv / (ms_k3 * 1e-3) / 1e12
    tiles = st["n_full"] + st["n_low"] + st["n_skip"] + st["n_skim"]
    counters = {} if args.low_refine else load_counters(args.workload)   # counters are of the E4M3 kernel

    # the plan (K1 + K2) as an HBM-bound pass: algorithmic bytes = read Q, K, V
    # (bf16) + E4M3 K and V + float32 means and scales (K1), + the means read
    # back, the int16 lists and the counts (K2), over the plan time
    N, d, H, Nq, Nk = cfg.seq_len, cfg.head_dim, cfg.heads * cfg.batch, cfg.n_qblocks, cfg.n_kblocks
    rb = (3 * N * d * H * 2 + 2 * N * d * H + (Nq + 2 * Nk) * d * H * 4 + 2 * Nk * H * 4
          + (Nq + Nk) * d * H * 4 + Nq * Nk * H * 2 + 12 * Nq * H)
    router = {"bytes_algorithmic": rb, "gb_s": round(rb / (ms_plan * 1e-3) / 1e9, 1),
              "frac_hbm": round(rb / (ms_plan * 1e-3) / 1e9 / PEAK_HBM, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(g, cfg, args.cpu_seconds, args.price)

    res = {
        "metric": "attention kernel ms + dense-equiv TFLOPS, 32760 tok x 40 heads x d128, 1 MI355X",
        "value": round(dense / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (dense-equivalent, plan + forward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16+fp8" + ("+fp4" if st["flops_fp4"] else "") + " (fp32 accumulate)",
        "data": "synthetic" + (f" ({args.gen_heads} generated heads tiled to {cfg.heads})" if tiled else ""),
        "config": {"workload": f"{cfg.name}: {cfg.grid[0]}x{cfg.grid[1]}x{cfg.grid[2]}={cfg.seq_len} tokens, "
                               f"{cfg.heads} heads, d={cfg.head_dim}, tiles {cfg.block_q}q x {cfg.block_k}k, "
                               + (f"tau_hi={cfg.tau_hi}, tau_lo={cfg.tau_lo}"
                                  + (f", tau_skim={cfg.tau_skim} (MXFP4 tier)" if cfg.tau_skim > 0 else "")
                                  if run_mode == "threshold" else
                                  f"price router, price={args.price}" if run_mode == "price" else
                                  f"entropy-adaptive k_h (keep {cfg.keep_min}-{cfg.keep_max}, FULL share "
                                  f"{cfg.full_frac}, {cfg.entropy_samples} sampled query blocks)"),
                   "batch": cfg.batch, "seq_len": cfg.seq_len, "heads": cfg.heads, "head_dim": cfg.head_dim},
        "kernel_ms": {"plan_k1_k2": round(ms_plan, 4), "forward_k3": round(ms_k3, 4),
                      "forward_k3_all_full": None if ms_allfull is None else round(ms_allfull, 4),
                      "replan_k1": round(ms_replan, 4), "step_with_plan_reuse": round(ms_reuse, 4),
                      "plan_median": round(med_plan, 4), "plan_min": round(min_plan, 4),
                      "forward_median": round(med_k3, 4), "forward_min": round(min_k3, 4)},
        "speedup_vs_all_full": None if ms_allfull is None else round(ms_allfull / ms_k3, 3),
        "forward_dense_equiv_tflops": round(dense / (ms_k3 * 1e-3) / 1e12, 2),
        "forward_executed_tflops": round(executed / (ms_k3 * 1e-3) / 1e12, 2),
        "mfma_utilisation_kept_tiles": round(achieved / PEAK_BF16, 4),
        "peak_fractions": {"forward_dense_equiv_of_bf16": round(dense / (ms_k3 * 1e-3) / 1e12 / PEAK_BF16, 4),
                           "forward_executed_of_bf16": round(executed / (ms_k3 * 1e-3) / 1e12 / PEAK_BF16, 4),
                           "forward_executed_of_fp8": round(executed / (ms_k3 * 1e-3) / 1e12 / PEAK_FP8, 4)},
        "router": router,
        "all_full_tflops": None if ms_allfull is None else round(dense / (ms_allfull * 1e-3) / 1e12, 2),
        "tiers": {"full": round(st["n_full"] / tiles, 4), "low": round(st["n_low"] / tiles, 4),
                  "skip": round(st["n_skip"] / tiles, 4), "diagonal": st["n_diag"],
                  **({"skim": round(st["n_skim"] / tiles, 4)} if st["n_skim"] else {}),
                  "near_threshold": n_band},
        "head_retention": kh_summary,
        "quality": quality,
        "skim_tier": skim_cmp,
        "low_refine": refine_cmp,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16, 4), "traffic": counters.get("bytes_per_launch"),
                     "kernel": "k3_attn (fused three-tier forward)",
                     "work": f"bf16 {st['flops_bf16'] / 1e12:.3f} TFLOP + fp8 {st['flops_fp8'] / 1e12:.3f} TFLOP "
                             f"(fp8 at the bf16/fp8 peak ratio, 1/2)"
                             + (f" + fp4 {st['flops_fp4'] / 1e12:.3f} TFLOP (fp4 at the bf16/fp4 peak ratio)"
                                if st["flops_fp4"] else "") + " per launch: U = frac",
                     "mfma_busy": counters.get("mfma_busy")},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
