"""Throughput of one MoE-layer training update (forward, backward, clip, AdamW)
on one MI355X, run as one persistent HIP kernel per update.

Prints ONE JSON line.  ``value`` is tokens/s over the timed updates with every
input resident in HBM; ``roofline`` relates the persistent kernel's average
launch time (HIP events on its own stream) to the update's algorithmic HBM
bytes; ``cpu_baseline`` is the FP64 oracle timed on this host's cores on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec per MoE-layer train update (fwd+bwd+AdamW); ms/update @2×1024"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_PEAK_TFLOPS = 157.3


def algorithmic_bytes(cfg, deferred=False) -> dict:
    """HBM bytes the update must move, phase by phase, with every cross-phase value
    stored once: token rows gathered into expert order, H and A in the activation
    dtype, expert outputs O in fp32, dO and dH and the per-slot input gradient in
    the activation dtype, fp32 gradients, 30 bytes per parameter for clip+AdamW
    (28 in fp32 mode).  Per microbatch unless marked.  With deferred weight
    gradients the expert gradients are written once per update, not once per
    microbatch."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, d, f, E, k = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k
    N = T * k
    W = E * d * f
    P = d * E + 2 * W
    ph = {
        "router_topk": T * d * es + d * E * 4 + T * k * 8,
        "gather": T * d * es + N * d * es,
        "ffn1": N * d * es + W * es + N * f * es,
        "ffn2": N * f * es + W * es + N * d * 4,
        "combine": N * d * 4 + T * d * es + N * d * es,
        "router_bwd": T * d * es,
        "dA_gelu": N * d * es + W * es + 2 * N * f * es,
        "dW2": N * f * es + N * d * es + W * 4,
        "dW1": N * d * es + N * f * es + W * 4,
        "dXs": N * f * es + W * es + N * d * es,
        "row_sum": N * d * es + T * d * 4,
    }
    per_mb = sum(ph.values())
    adamw = P * (30 if cfg.dtype == "bf16" else 28)
    per_update = per_mb * cfg.microbatches + adamw
    if deferred:
        per_update -= 2 * W * 4 * (cfg.microbatches - 1)
    return {"per_microbatch": per_mb, "adamw": adamw, "per_update": per_update, "phases": ph}


PROFILE_DIR = os.path.join(ROOT, "profiles")


def kernel_source_sha256() -> str:
    """Hash of the sources the persistent kernel is built from (the same recipe
    as the one recorded with the counter profile)."""
    import glob
    import hashlib
    files = sorted(glob.glob(os.path.join(ROOT, "moe_step_megakernel_amd", "csrc", "*.h"))
                   + [os.path.join(ROOT, "moe_step_megakernel_amd", "csrc", "moe_step.hip"),
                      os.path.join(ROOT, "include", "moe_step.h")],
                   key=lambda f: os.path.relpath(f, ROOT))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cfg):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE profile of
    this workload, scaled by the copy calibration; None if there is none or the
    kernel sources changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"moe_step_kernel_{cfg.name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        doc = json.load(fh)
    if doc.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return float(doc["hbm_bytes_per_launch"])


def gemm_flops(cfg) -> int:
    return 6 * 2 * cfg.tokens * cfg.top_k * cfg.d_model * cfg.d_ff * cfg.microbatches


def cpu_baseline(cfg, inp, budget_s: float, one_thread: bool = True) -> dict:
    """The oracle as it stands, on this host's cores, repeated over the same batch
    until about ``budget_s`` seconds of work (at least one update); then, for
    scale, one more update on a single BLAS thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    params = inp.flat_params().astype(np.float64)
    m = np.zeros_like(params)
    v = np.zeros_like(params)
    xs = [inp.microbatch(i)[0] for i in range(cfg.microbatches)]
    ts = [inp.microbatch(i)[1] for i in range(cfg.microbatches)]
    reps, t0 = 0, time.perf_counter()
    while True:
        out = oracle.step(xs, ts, params, m, v, reps + 1, d=cfg.d_model, f=cfg.d_ff, E=cfg.n_experts,
                          top_k=cfg.top_k, lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                          weight_decay=cfg.weight_decay, clip_norm=cfg.clip_norm, bias=inp.router_bias)
        params, m, v = out["params"], out["exp_avg"], out["exp_avg_sq"]
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    tok = cfg.tokens_in_update * reps
    res = {"value": tok / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{reps} full FP64 update(s) of the {cfg.name} layer ({cfg.tokens_in_update} tokens each), "
                     f"{el:.1f} s", "ms_per_update": 1e3 * el / reps}
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        res["blas"] = ",".join(sorted({str(i.get("internal_api")) for i in threadpool_info()
                                       if i.get("user_api") == "blas"})) or None
        # one update on a single BLAS thread, for scale
        if one_thread:
            with threadpool_limits(limits=1, user_api="blas"):
                t1 = time.perf_counter()
                oracle.step(xs, ts, params, m, v, reps + 1, d=cfg.d_model, f=cfg.d_ff, E=cfg.n_experts,
                            top_k=cfg.top_k, lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                            weight_decay=cfg.weight_decay, clip_norm=cfg.clip_norm, bias=inp.router_bias)
                res["ms_per_update_1_thread"] = 1e3 * (time.perf_counter() - t1)
    except Exception:  # pragma: no cover - threadpoolctl missing or refusing
        pass
    return res


def bench_selective(args, cfg, layer, X, Tg, bias, dx, stream):
    """Selective updates (the pages' "Other measured compiler work" table: shared
    weights every microbatch, experts every 16): one launch per microbatch of
    cfg.tokens tokens, router clip+AdamW in every launch, expert gradients
    accumulated over W launches and applied in the last."""
    import torch

    W = args.selective
    T = cfg.tokens
    n = [0]

    def one_microbatch(ev=None):
        i = n[0]
        n[0] += 1
        groups = dict(zero_router=True, apply_router=True, step_router=i + 1, zero_experts=(i % W == 0),
                      apply_experts=(i % W == W - 1), step_experts=i // W + 1)
        if ev is not None:
            ev[0].record(stream)
        layer.run(X[:T], Tg[:T], tokens_in_update=T, dx=dx, router_bias=bias, groups=groups)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(W * max(1, -(-args.warmup // W))):
        one_microbatch()
    torch.cuda.synchronize()
    layer.status()
    steps = W * max(1, -(-args.steps // W))   # whole windows
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        one_microbatch(ev[i])
    t1.record(stream)
    torch.cuda.synchronize()
    layer.status()
    total_ms = t0.elapsed_time(t1)
    ms = np.array([s.elapsed_time(e) for s, e in ev])
    per_pos = [float(np.median(ms[j::W])) for j in range(W)]
    layer.close()
    line = {
        "metric": f"ms per microbatch, selective updates (router every microbatch, experts every {W})",
        "value": T * steps / (total_ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": W * max(1, -(-args.warmup // W)), "ms_per_step": total_ms / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"MoE-FFN layer {cfg.name}, {T}-token microbatches, d_model={cfg.d_model}, "
                               f"d_ff={cfg.d_ff}, E={cfg.n_experts}, top-{cfg.top_k}, expert window {W}",
                   "tokens_per_microbatch": T, "parallelism": "single-gpu"},
        "ms_per_microbatch_median": float(np.median(ms)),
        "ms_router_only_microbatch_median": float(np.median(np.concatenate([ms[j::W] for j in range(W - 1)])))
        if W > 1 else None,
        "ms_expert_update_microbatch_median": per_pos[-1],
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="bf16_2x1024")
    ap.add_argument("--wg-per-cu", type=int, default=0)
    ap.add_argument("--cooperative", action="store_true",
                    help="launch through hipLaunchCooperativeKernel instead of an ordinary launch")
    ap.add_argument("--ready-gemm12", action="store_true",
                    help="per-row-tile readiness counters instead of the grid barrier between the expert products")
    ap.add_argument("--barrier-per-workgroup", action="store_true",
                    help="every workgroup writes its XCD's L2 back at each grid barrier (instead of one per XCD)")
    ap.add_argument("--recompute", action="store_true",
                    help="memory rule: store H only and recompute gelu(H) / gelu'(H) where they are read")
    ap.add_argument("--no-defer", action="store_true",
                    help="updates over several microbatch launches add their expert weight gradients every "
                         "launch instead of deferring them to the applying launch")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--dump-trace", default=None, help="write the raw phase clocks (.npy) here")
    ap.add_argument("--selective", type=int, default=0, metavar="W",
                    help="time selective updates instead: the router is updated after every microbatch, the "
                         "experts after every W (one timed step = one microbatch)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              f"(the update's multi-GPU sharding is described, not built)", file=sys.stderr)
        return 2

    import torch

    import synth
    from moe_step_megakernel_amd import trace as trace_mod
    from moe_step_megakernel_amd.layer import MoeLayerStep

    cfg = synth.CONFIGS[args.config]
    print(f"# bench {cfg.name}: T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} "
          f"E={cfg.n_experts} k={cfg.top_k} {cfg.dtype}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, 0)
    dev = torch.device("cuda", 0)
    # updates over several microbatch launches defer the expert weight
    # gradients to the applying launch (bf16, plain updates) unless told not to
    defer = cfg.microbatches if (cfg.microbatches > 1 and cfg.dtype == "bf16" and not args.recompute
                                 and args.selective == 0 and not args.no_defer) else 0
    layer = MoeLayerStep(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, cfg.tokens, cfg.dtype, lr=cfg.lr,
                         beta1=cfg.beta1, beta2=cfg.beta2, adam_eps=cfg.eps, weight_decay=cfg.weight_decay,
                         clip_norm=cfg.clip_norm, wg_per_cu=args.wg_per_cu,
                         memory_rules=1 if args.recompute else 0, max_microbatches=defer)
    layer.load_params(torch.from_numpy(inp.flat_params()))

    def tok(a, bits):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    X, Tg = tok(inp.x, inp.x_bits), tok(inp.t, inp.t_bits)
    bias = None if inp.router_bias is None else torch.from_numpy(inp.router_bias).to(dev)
    dx = torch.empty(cfg.tokens, cfg.d_model, dtype=torch.float32, device=dev)
    T, M = cfg.tokens, cfg.microbatches
    stream = torch.cuda.current_stream(dev)
    step_no = [0]

    def one_update(events=None, trace=None):
        step_no[0] += 1
        for mb in range(M):
            if events is not None:
                events[mb][0].record(stream)
            layer.run(X[mb * T:(mb + 1) * T], Tg[mb * T:(mb + 1) * T], tokens_in_update=cfg.tokens_in_update,
                      step=step_no[0], zero_grad=(mb == 0), apply=(mb == M - 1), dx=dx, router_bias=bias,
                      trace=trace, ready_gemm12=args.ready_gemm12, cooperative=args.cooperative,
                      barrier_per_workgroup=args.barrier_per_workgroup)
            if events is not None:
                events[mb][1].record(stream)

    if args.selective > 0:
        return bench_selective(args, cfg, layer, X, Tg, bias, dx, stream)

    # pristine state for the "fresh" clock: the first update's routing
    pristine = (layer.params.clone(), layer.exp_avg.clone(), layer.exp_avg_sq.clone())
    for _ in range(args.warmup):
        one_update()
    torch.cuda.synchronize()
    layer.status()

    # the timed region: K updates back to back between two events on the launch
    # stream (nothing else enqueued between the launches)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        one_update()
    t_end.record(stream)
    torch.cuda.synchronize()
    layer.status()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    value = cfg.tokens_in_update * args.steps / (total_ms / 1e3)
    # the spread: another K updates with events around every launch (the
    # events add a few microseconds between launches, so they stay out of the
    # timed region)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(M)]
          for _ in range(args.steps)]
    for i in range(args.steps):
        one_update(ev[i])
    torch.cuda.synchronize()
    layer.status()
    launch_ms = np.array([[s.elapsed_time(e) for s, e in row] for row in ev])
    upd_ms = launch_ms.sum(axis=1)
    print(f"# {args.steps} updates in {total_ms:.3f} ms; per update (separate pass) median {np.median(upd_ms):.4f} ms "
          f"p10 {np.percentile(upd_ms, 10):.4f} p90 {np.percentile(upd_ms, 90):.4f}", file=sys.stderr, flush=True)

    # fresh clock: params and moments restored from the pristine copy before
    # each timed update (outside its events), so every one routes like the
    # first; the bf16 weight copy is not restored (its values do not change the
    # work), the continuing-training clock above keeps evolving the state
    fresh_ms = []
    saved = (layer.params.clone(), layer.exp_avg.clone(), layer.exp_avg_sq.clone(), step_no[0])
    for _ in range(min(args.steps, 20)):
        for dst, src in zip((layer.params, layer.exp_avg, layer.exp_avg_sq), pristine):
            dst.copy_(src)
        step_no[0] = 0
        ev_f = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(M)]
        one_update(ev_f)
        torch.cuda.synchronize()
        fresh_ms.append(float(sum(s.elapsed_time(e) for s, e in ev_f)))
    for dst, src in zip((layer.params, layer.exp_avg, layer.exp_avg_sq), saved[:3]):
        dst.copy_(src)
    step_no[0] = saved[3]
    torch.cuda.synchronize()
    layer.status()
    del pristine, saved
    print(f"# fresh-state updates: median {np.median(fresh_ms):.4f} ms", file=sys.stderr, flush=True)

    phases = None
    if not args.no_trace:
        words = layer.trace_words()
        tr = torch.zeros(words, dtype=torch.int64, device=dev)
        # a few traced updates: the overhead figure is their median launch time
        # against the untraced median; the clocks decoded are the last one's
        traced_ms = []
        for _ in range(5):
            ev_tr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(M)]
            one_update(ev_tr, trace=tr)
            torch.cuda.synchronize()
            traced_ms.append(float(ev_tr[-1][0].elapsed_time(ev_tr[-1][1])))
        layer.status()
        raw = tr.cpu().numpy()
        if args.dump_trace:
            np.save(args.dump_trace, raw.reshape(layer.grid, -1, 3))
        phases = trace_mod.decode(raw, layer.grid)
        phases["traced_launch_ms"] = float(np.median(traced_ms))
        phases["trace_overhead_frac"] = phases["traced_launch_ms"] / float(np.median(launch_ms[:, -1])) - 1.0
        print("# phases (us): " + " ".join(f"{k}={v:.1f}" for k, v in phases["phase_us"].items())
              + f"  barrier idle mean {phases['barrier_idle_frac_mean']:.3f}", file=sys.stderr, flush=True)

    ab = algorithmic_bytes(cfg, deferred=defer > 0)
    # the dominant (and only) kernel: one launch per microbatch, its average
    # duration from the timed region (bytes: the update's, averaged over its launches)
    avg_launch_s = total_ms / (args.steps * M) / 1e3
    bytes_per_launch = ab["per_update"] / M
    achieved = bytes_per_launch / avg_launch_s / 1e9
    traffic = measured_traffic(cfg)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": "moe::moe_step_kernel (persistent, one launch per update)", "workgroups": layer.grid,
                "launch": "cooperative" if args.cooperative else "ordinary",
                "algorithmic_bytes_per_launch": int(bytes_per_launch),
                "avg_launch_us": avg_launch_s * 1e6,
                "gemm_tflops_effective": gemm_flops(cfg) / M / avg_launch_s / 1e12}

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the FP64 oracle on the host ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, inp, args.cpu_budget)

    arena_bytes = layer.arena_bytes()
    layer.close()
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"MoE-FFN layer update {cfg.name}: {cfg.tokens}x{cfg.microbatches} tokens, "
                               f"d_model={cfg.d_model}, d_ff={cfg.d_ff}, E={cfg.n_experts}, top-{cfg.top_k}",
                   "tokens_per_update": cfg.tokens_in_update, "global_batch": cfg.tokens_in_update,
                   "seq_len": 1024, "parallelism": "single-gpu",
                   **({"ready_gemm12": True} if args.ready_gemm12 else {}),
                   **({"memory_rules": "recompute"} if args.recompute else {}),
                   **({"deferred_weight_gradients": defer} if defer else {})},
        "ms_per_update_median": float(np.median(upd_ms)), "ms_per_update_p10": float(np.percentile(upd_ms, 10)),
        "ms_per_update_p90": float(np.percentile(upd_ms, 90)),
        "ms_per_update_fresh_median": float(np.median(fresh_ms)),
        "roofline": roofline, "cpu_baseline": cpu, "phases": phases, "arena_bytes": arena_bytes,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
