"""Benchmark: useful partial-attention TFLOP/s on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the partial-attention layer call (npa_attn_fwd) and
the structure-guidance blend (npa_sg_blend) of the workload.  First --settle
seconds of back-to-back steps (the GPU's clock governor raises the shader
clock over a second or two of sustained load), then W untimed warm-up steps,
then K steps timed with HIP events on the stream the kernels run on.

The JSON line carries:
  value     -- useful attention flops per step / step time (TFLOP/s);
  roofline  -- the attention kernel alone: useful flops / its average launch
               duration (HIP events around each launch), against the dense
               bf16 MFMA peak at 2.4 GHz; sclk_mhz / power_w are the shader
               clock and board power sampled from sysfs during the timed
               steps, frac_at_sclk the fraction of the peak at that clock;
  cpu_baseline -- the fp64 oracle timed on a bounded sample of the same
               workload on this host's cores (rank 0, N=1 only); its
               "tier0" entry times the oracle's brute-force loops on a
               bounded sample of the tiny fp32 strip layer;
  also       -- the other 4096^2 layer (FLUX-shaped, head_dim 128, when the
               headline workload is the SDXL one), timed in the same process:
               its attention kernel's launches, with the same roofline fields.
  roofline.measured_mfma_ceiling -- after the timed steps, a dense
               v_mfma_f32_16x16x32_bf16 stream (the kernel's instruction) on random and on constant
               operands: what this GPU sustains under its clock and power
               management (the published peak assumes 2.4 GHz throughout).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Dense bf16 MFMA peak of MI355X: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
# Dense fp32 MFMA peak of MI355X (the fp32 kernel runs on v_mfma_f32_16x16x4_f32).
PEAK_F32_MFMA_TFLOPS = 157.3
GRAPH_TIMING = ("100 launches replayed from one HIP graph; the inputs stay resident in the GPU's caches "
                "between launches, so this is a cache-resident rate, not an HBM one")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(name: str, inp: dict, budget_s: float) -> dict:
    """The oracle (as it is) on whole query tiles, (batch, head) pair after pair,
    until the time budget is spent; the rate is its useful flops per second."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    from partial_context_patch_amd import workloads as WL

    w = WL.ATTENTION_WORKLOADS[name]
    spec = (A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows")) if w["mode"] == "strips"
            else A.Windows(w["tile_h"], w["tile_w"], w["halo_h"], w["halo_w"], w.get("text_tokens", 0)))
    H, W, d = w["map_h"], w["map_w"], w["head_dim"]
    tiles = list(A.iter_tiles(H, W, spec))
    done_pairs, n_tiles, t0 = 0, 0, time.perf_counter()
    heads = [(b, j) for b in range(w["batch"]) for j in range(w["heads"])]
    for b, j in heads:
        for qt, ft, st in tiles:
            A.attention_tier1(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec,
                              query_tokens=qt, heads=[(b, j)])
            done_pairs += len(qt) * (len(ft) + len(st))
            n_tiles += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {
        "value": 4 * d * done_pairs / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_tiles} (batch, head, query tile) units of {len(tiles) * len(heads)} "
                  f"({done_pairs} attended pairs, {4 * d * done_pairs / 1e9:.1f} useful GFLOP) in {secs:.1f} s; "
                  f"fp64 numpy, BLAS threads={threads}, host cpus={os.cpu_count()}, cpu: {cpu_model()}",
    }


def cpu_tier0(budget_s: float = 6.0) -> dict:
    """The oracle's brute-force tier (Python loops over every query, key and
    channel, key sets from the per-pair predicate) on a bounded sample of the
    tiny fp32 strip layer: queries spread over its strips, one (batch, head)
    pair; the rate is useful flops of the sampled pairs per second, the time
    including the key-set enumeration."""
    import numpy as np

    from oracle import attention as A
    from partial_context_patch_amd import workloads as WL

    name = "pcpp_tiny_fp32"
    w = WL.ATTENTION_WORKLOADS[name]
    spec = A.Strips(w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
    H, W, d = w["map_h"], w["map_w"], w["head_dim"]
    inp = WL.workload_inputs(name)
    tiles = list(A.iter_tiles(H, W, spec))
    size = {int(t): len(ft) + len(st) for qt, ft, st in tiles for t in qt}
    n = 8
    while True:
        qs = np.linspace(0, H * W - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        A.attention_tier0(inp["q"], inp["k"], inp["v"], inp["k_stale"], inp["v_stale"], H, W, spec,
                          query_tokens=qs, heads=[(0, 0)])
        secs = time.perf_counter() - t0
        if secs >= budget_s / 3 or n >= H * W:
            break
        n = min(H * W, n * 4)
    pairs = sum(size[int(t)] for t in qs)
    return {"value": 4 * d * pairs / secs / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"tier 0 (Python loops) on {name}: {len(qs)} of {H * W} queries, 1 of "
                      f"{w['batch'] * w['heads']} (batch, head) pairs ({pairs} attended pairs) in {secs:.2f} s"}


def mfma_ceiling():
    """Run the dense-MFMA calibration program (a child process; about 3 s) and
    return its measurements, or None when it is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "partial_context_patch_amd", "calib", "mfma_ceiling")
    if not os.path.exists(exe):
        log("mfma ceiling: calibration program not built")
        return None
    log("measuring the dense bf16 MFMA ceiling (random and constant operands)")
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        log("mfma ceiling: timed out")
        return None
    if r.returncode != 0:
        log(f"mfma ceiling: failed ({r.stderr.strip()[-200:]})")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sdxl4096_npa")
    ap.add_argument("--dtype", choices=("bf16", "f32"), default=None,
                    help="run the workload's shape in this dtype instead of its own (f32: the fp32 path; "
                         "bf16 head sizes are 64 and 128)")
    ap.add_argument("--also", default=None,
                    help="another attention workload whose kernel launches are timed in the same process "
                         "(default: the FLUX-shaped 4096^2 layer when the headline is the SDXL one; 'none' skips)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--settle", type=float, default=3.0,
                    help="seconds of back-to-back steps before the warm-up steps, so that the GPU's clock "
                         "governor has raised the shader clock to its sustained level (it ramps over ~1-2 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the dense-MFMA calibration run (after the timed steps) that measures the "
                         "bf16 MFMA throughput this GPU sustains on random and on constant operands")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (outside the timed region) so that a "
                         "counter profile of this command can scale its byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the partial-attention kernels run and are timed on a single MI355X; "
              "multi-GPU runs are not supported (the path would shard by (batch, head, tile) units, or by strips "
              "with a stale-halo exchange between neighbouring GPUs).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from partial_context_patch_amd import npa, profiling
    from partial_context_patch_amd import workloads as WL

    npa.load()  # builds the library in-tree only when none is built
    name = args.workload
    also = args.also
    if also is None:
        also = "flux4096_npa" if name == "sdxl4096_npa" else "none"
    sgw = WL.SG_WORKLOAD
    dev = torch.device("cuda:0")
    x, ref = WL.sg_inputs(sgw["channels"], sgw["map_h"], sgw["map_w"], seed=sgw["seed"])
    x, ref = torch.from_numpy(x).to(dev), torch.from_numpy(ref).to(dev)
    sg_out = torch.empty_like(x)

    if args.copy_calibration:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 512 MiB read + 512 MiB written")
        del src, dst

    def layer(wname, dtype, with_sg):
        """Time one attention workload: settle, warm up, then K timed steps
        (attention, plus the SG blend when with_sg), HIP events around each
        launch on the stream the kernels run on."""
        w = WL.ATTENTION_WORKLOADS[wname]
        if dtype is not None:
            w = dict(w, dtype=dtype)
        log(f"workload {wname} ({w['dtype']}): {w['what']}")
        inp = WL.attention_inputs(**w, stale=(w["mode"] == "strips"))
        tdt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
        t = {n: (None if a is None else torch.from_numpy(a).to(dev).to(tdt)) for n, a in inp.items()}
        out = torch.empty_like(t["q"])
        kw = WL.halo_kwargs(w)
        L = npa.make_layout(w["batch"], w["heads"], w["head_dim"], w["map_h"], w["map_w"], dtype=w["dtype"])
        flops = npa.useful_flops(L, npa.make_halo(**kw))
        hw = (w["map_h"], w["map_w"])

        def step(ev=None):
            if ev is not None:
                ev[0].record()
            npa.attn_fwd(t["q"], t["k"], t["v"], t["k_stale"], t["v_stale"], map_hw=hw, out=out, **kw)
            if ev is not None:
                ev[1].record()
            if with_sg:
                npa.sg_blend(x, ref, sgw["w_t"], sgw["sigma"], out=sg_out)
            if ev is not None:
                ev[2].record()

        # settle: the shader clock ramps up over a second or two of sustained
        # load; a diffusion sampler keeps the GPU busy for far longer than that,
        # so steps are timed at the sustained clock
        # (batches of 10 steps; the host waits on the batch before the last one,
        # so the GPU's queue never runs dry and the clock sees no idle gaps)
        t_settle = time.perf_counter()
        n_settle = 0
        pending = []
        while time.perf_counter() - t_settle < args.settle:
            for _ in range(10):
                step()
            n_settle += 10
            e = torch.cuda.Event()
            e.record()
            pending.append(e)
            if len(pending) > 2:
                pending.pop(0).synchronize()
        if args.settle > 0:
            log(f"settled the clock with {n_settle} steps in {time.perf_counter() - t_settle:.1f} s")
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # the GPU's shader clock and board power, sampled from sysfs while the
        # timed steps run; started before the synchronisation below, so that
        # nothing but the launch latency separates the last warm-up step from the
        # first timed one (after an idle gap of a few ms the clock governor takes
        # several launches to come back to its sustained level)
        sampler = profiling.ClockSampler().start()
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(evs[i])
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        sampler.stop()
        clock = sampler.summary()
        ms_step = start.elapsed_time(stop) / args.steps
        attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
        sg_ms = [e[1].elapsed_time(e[2]) for e in evs]
        attn_avg = float(np.mean(attn_ms))
        p10, med, p90 = (float(v) for v in np.percentile(attn_ms, [10, 50, 90]))
        log(f"{wname}: step {ms_step:.4f} ms (wall {wall * 1e3 / args.steps:.4f} ms); attention avg "
            f"{attn_avg:.4f} ms p10 {p10:.4f} median {med:.4f} p90 {p90:.4f} min {min(attn_ms):.4f} "
            f"max {max(attn_ms):.4f}")
        bf16 = w["dtype"] == "bf16"
        peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_MFMA_TFLOPS
        achieved = flops / (attn_avg * 1e-3) / 1e12
        sclk = clock.get("sclk_mhz")
        traffic = profiling.load_traffic(wname) if bf16 else None
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None if traffic is None else int(traffic),
                "kernel": "attn_bf16_kernel" if bf16 else "attn_f32_kernel", "avg_launch_ms": round(attn_avg, 5),
                "launch_ms_p10_median_p90": [round(p10, 5), round(med, 5), round(p90, 5)],
                "sclk_mhz": sclk, "sclk_samples": clock["sclk_samples"],
                "power_w": clock["power_w"], "power_cap_w": clock["power_cap_w"],
                "frac_at_sclk": None if not sclk else round(achieved / (peak * sclk / 2400.0), 4),
                "watts_per_useful_tflops": (round(clock["power_w"] / achieved, 4)
                                            if clock.get("power_w") and achieved > 0 else None)}
        cfg = {"workload": wname, "what": w["what"], "batch": w["batch"], "heads": w["heads"],
               "head_dim": w["head_dim"], "map": f"{w['map_h']}x{w['map_w']}", "useful_gflop_per_step": flops / 1e9}
        if w["mode"] == "strips":
            cfg.update(strips=w["num_strips"], p=w.get("p"), halo_rows=w.get("halo_rows"))
        else:
            cfg.update(tile=f"{w['tile_h']}x{w['tile_w']}", halo=w["halo_h"])
            if w.get("text_tokens"):
                cfg.update(text_tokens=w["text_tokens"])
        res = dict(w=w, inp=inp, flops=flops, ms_step=ms_step, sg_avg=float(np.mean(sg_ms)), roof=roof, cfg=cfg)
        del t, out
        torch.cuda.synchronize()
        return res

    main_res = layer(name, args.dtype, True)
    w = main_res["w"]
    ms_step = main_res["ms_step"]
    value = main_res["flops"] / (ms_step * 1e-3) / 1e12
    # structure-guidance blend: reads x and ref, writes out, 4 bytes each per element
    sg_bytes = 12 * sgw["channels"] * sgw["map_h"] * sgw["map_w"]

    # The blend is a few-microsecond kernel: an event pair around each launch adds
    # microseconds to it, and a Python loop of launches cannot issue them that fast.  So it is
    # also timed as 100 launches captured in one HIP graph, replayed between two
    # events.  An elementwise op that moves the same bytes (x + ref: reads both,
    # writes one array), timed the same way, gives the streaming floor of a
    # launch of this size.
    def graph_ms(fn, n=100):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    sg_loop = graph_ms(lambda: npa.sg_blend(x, ref, sgw["w_t"], sgw["sigma"], out=sg_out))
    floor_ms = graph_ms(lambda: torch.add(x, ref, out=sg_out))
    # the asynchronous structure-guidance correction on a latent of the same
    # shape (not part of the step): 16 bytes per element (eps, eps_ref_prev and
    # mask read, out written), in place on eps as a sampler would run it
    eps, eps_ref, mask = (torch.from_numpy(a).to(dev) for a in WL.asg_inputs(tuple(x.shape), seed=sgw["seed"] + 1))
    asg_ms = graph_ms(lambda: npa.asg_blend(eps, eps_ref, mask, 0.5, out=eps))
    asg_bytes = 16 * x.numel()

    also_rec = None
    if also != "none" and also != name:
        r = layer(also, None, False)
        also_rec = dict(r["cfg"], roofline=r["roof"])

    ceiling = None
    if not args.no_mfma_ceiling:
        ceiling = mfma_ceiling()
    for roof in [main_res["roof"]] + ([also_rec["roofline"]] if also_rec else []):
        roof["measured_mfma_ceiling"] = ceiling
        roof["frac_of_measured_ceiling"] = (round(roof["achieved"] / ceiling["random_tflops"], 4)
                                            if roof["kernel"] == "attn_bf16_kernel" and ceiling
                                            and ceiling.get("random_tflops") else None)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample of the same workload")
        cpu = cpu_baseline(name, main_res["inp"], args.cpu_budget)
        log("timing the oracle's brute-force tier on a bounded sample of the tiny strip layer")
        cpu["tier0"] = cpu_tier0()

    cfg = dict(main_res["cfg"], sg_blend=sgw["what"])
    rec = {
        "metric": "useful partial-attention TFLOP/s & % of bf16 MFMA peak per denoise step",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "dtype": w["dtype"],
        "data": "synthetic (seeded N(0,1) activations of the workload's shape; no weights or datasets)",
        "config": cfg,
        "roofline": main_res["roof"],
        "sg_blend": {"bound": "hbm", "achieved": round(sg_bytes / (sg_loop * 1e-3) / 1e9, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(sg_bytes / (sg_loop * 1e-3) / 1e9 / 8000.0, 4),
                     "algorithmic_bytes": sg_bytes, "avg_launch_ms": round(sg_loop, 5),
                     "in_step_event_ms": round(main_res["sg_avg"], 5),
                     "same_bytes_elementwise_ms": round(floor_ms, 5),
                     "frac_of_same_bytes": round(floor_ms / sg_loop, 4), "timing": GRAPH_TIMING},
        "asg_blend": {"bound": "hbm", "achieved": round(asg_bytes / (asg_ms * 1e-3) / 1e9, 1), "peak": 8000.0,
                      "unit": "GB/s", "frac": round(asg_bytes / (asg_ms * 1e-3) / 1e9 / 8000.0, 4),
                      "algorithmic_bytes": asg_bytes, "avg_launch_ms": round(asg_ms, 5), "timing": GRAPH_TIMING},
        "also": also_rec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
