"""Per-phase profile of the persistent update kernel on one workload, from
rocprofv3 runs of the C++ driver of the C ABI (``_lib/moe_step_bench``) on the
exact seeded inputs of the tests (``synth.dump``).

    python -m moe_step_megakernel_amd.profile --config NAME [--steps K] [--warmup W]
           [--fresh] [--work DIR] [--out profiles]

With --fresh every update starts from the initial parameters and zero moments
(``moe_step_bench --fresh``), so each one routes like the first; without it
the parameters keep training over the run, which moves the routing of a
skewed workload towards balance as the masks go by.

Runs, each as its own process (the profiler starts the driver itself):

1. uncounted timing of every skip mask (``moe_step_bench --skip``): each phase
   alone (every other phase skipped; the grid barriers and the route_order
   offsets always run, the "skeleton"), plus the dispatch gather and the k-way
   row sum of dx on their own (the same phase with and without that step);
2. ``rocprofv3 --kernel-trace --stats`` of full updates;
3. two counter passes over the same masks: MFMA instructions, MFMA busy cycles,
   GPU-active cycles and FETCH_SIZE; then WRITE_SIZE;
4. the same two memory counters for a plain device copy of 256 MiB (read and
   write), which scales FETCH_SIZE / WRITE_SIZE to bytes.

Writes ``moe_step_kernel_<config>_phases.md`` (table and commands),
``moe_step_kernel_<config>_kernel_trace.md`` (the stats of run 2) and
``moe_step_kernel_<config>_hbm_traffic.json`` (bytes per launch of full
updates, with the hash of the kernel sources) into the output directory.
This module starts programs and reads their files; it never touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BENCH = os.path.join(HERE, "_lib", "moe_step_bench")
HBM_PEAK = 8.0e12
BF16_PEAK = 2.5e15

# (label, mask, baseline label): phase cost = launch(mask) - launch(baseline)
MASKS = [
    ("skeleton (barriers, route_order offsets)", 0x0FF, None),
    ("route: W_r copy, logits, top-k, gates, histogram", 0x0FE, "skeleton (barriers, route_order offsets)"),
    ("route_order scatter + dispatch gather", 0x0FD, "skeleton (barriers, route_order offsets)"),
    ("route_order scatter alone", 0x1FD, "skeleton (barriers, route_order offsets)"),
    ("GEMM 1 + GELU", 0x0FB, "skeleton (barriers, route_order offsets)"),
    ("GEMM 2", 0x0F7, "skeleton (barriers, route_order offsets)"),
    ("combine, loss, dO, dz", 0x0EF, "skeleton (barriers, route_order offsets)"),
    ("dH + dW2 + router partials", 0x0DF, "skeleton (barriers, route_order offsets)"),
    ("dW1 + dX + router gradient", 0x0BF, "skeleton (barriers, route_order offsets)"),
    ("dx row sum + norm + clip/AdamW", 0x07F, "skeleton (barriers, route_order offsets)"),
    ("norm + clip/AdamW alone", 0x27F, "skeleton (barriers, route_order offsets)"),
    ("full update", 0x000, None),
]
# steps measured as a difference of two masks
DIFFS = [
    ("dispatch gather (S4)", "route_order scatter + dispatch gather", "route_order scatter alone"),
    ("k-way row sum of dx (S13)", "dx row sum + norm + clip/AdamW", "norm + clip/AdamW alone"),
]
PASS_A = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "FETCH_SIZE"]
PASS_B = ["WRITE_SIZE"]


def log(*a):
    print("[profile]", *a, flush=True)


def kernel_source_sha256() -> str:
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h"))
                   + [os.path.join(HERE, "csrc", "moe_step.hip"), os.path.join(ROOT, "include", "moe_step.h")],
                   key=lambda f: os.path.relpath(f, ROOT))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def shown(cmd) -> str:
    """A command as printed in the summaries: paths inside the repository as <repo>/..."""
    return " ".join(cmd).replace(ROOT, "<repo>")


def run(cmd, timeout):
    log("$ " + " ".join(cmd))
    res = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"exit {res.returncode}: {' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}")
    return res.stdout


def find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def moe_dispatch_counters(path):
    """{dispatch id: {counter: value}} for the update kernel, in dispatch order."""
    out = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if "moe_step_kernel" not in row.get("Kernel_Name", ""):
                continue
            did = int(row["Dispatch_Id"])
            out.setdefault(did, {})
            out[did][row["Counter_Name"]] = out[did].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [out[k] for k in sorted(out)]


def copy_dispatch_counters(path):
    """The same for the driver's copy kernel."""
    out = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if "copy_kernel" not in row.get("Kernel_Name", ""):
                continue
            did = int(row["Dispatch_Id"])
            out.setdefault(did, {})
            out[did][row["Counter_Name"]] = out[did].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [out[k] for k in sorted(out)]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", required=True)
    ap.add_argument("--steps", type=int, default=5, help="updates per mask")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--timing-steps", type=int, default=30, help="updates per mask in the uncounted timing run")
    ap.add_argument("--work", default=os.path.join(tempfile.gettempdir(), "moe_step_prof"),
                    help="directory for the raw rocprofv3 output")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--inputs-dir", default="/tmp")
    ap.add_argument("--fresh", action="store_true",
                    help="every update from the initial parameters and zero moments (the routing of the first)")
    ap.add_argument("--defer", action="store_true",
                    help="deferred expert weight gradients (max_microbatches = the update's microbatches)")
    args = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import synth
    from synth import dump as synth_dump

    cfg = synth.CONFIGS[args.config]
    work = os.path.abspath(os.path.join(args.work, args.config))
    os.makedirs(work, exist_ok=True)
    os.makedirs(args.out, exist_ok=True)
    inputs = os.path.join(args.inputs_dir, f"moe_profile_inputs_{cfg.name}.bin")   # large: kept out of work
    synth_dump.dump(cfg, 0, inputs)
    log(f"inputs of {cfg.name} written to {inputs}")
    masks = ",".join(f"0x{m:03x}" for _, m, _ in MASKS)
    drv = [BENCH, "--inputs", inputs, "--warmup", str(args.warmup)] + (["--fresh"] if args.fresh else []) + \
        (["--defer"] if args.defer else [])
    M = cfg.microbatches

    # 1. uncounted timing
    out = run(drv + ["--steps", str(args.timing_steps), "--skip", masks], 600)
    ms = {}
    grid = None
    for line in out.splitlines():
        m = re.search(r"skip=0x([0-9a-f]+) grid=(\d+): .* ([0-9.]+) ms/update", line)
        if m:
            ms[int(m.group(1), 16)] = float(m.group(3))
            grid = int(m.group(2))
    log("timing (ms/update): " + " ".join(f"0x{k:03x}={v:.4f}" for k, v in ms.items()))

    # 2. kernel trace + stats of full updates
    kt_dir = os.path.join(work, "kernel_trace")
    kt_cmd = ["rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d", kt_dir, "-o", "kt", "--"] + drv + \
        ["--steps", str(args.timing_steps), "--skip", "0"]
    run(kt_cmd, 300)
    stats_rows = list(csv.DictReader(open(find(kt_dir, "kernel_stats.csv"))))
    trace_rows = [r for r in csv.DictReader(open(find(kt_dir, "kernel_trace.csv")))
                  if "moe_step_kernel" in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace_rows]
    timed = durs[args.warmup * M:]
    log(f"kernel trace: {len(durs)} launches, timed mean {sum(timed) / max(1, len(timed)):.1f} us")

    # 3. counters per mask; 4. copy calibration
    def pmc(counters, tag, cmd):
        d = os.path.join(work, tag)
        run(["rocprofv3", "--pmc", *counters, "-f", "csv", "-d", d, "-o", "pmc", "--"] + cmd, 300)
        return find(d, "counter_collection.csv")

    pa = moe_dispatch_counters(pmc(PASS_A, "pmcA", drv + ["--steps", str(args.steps), "--skip", masks]))
    pb = moe_dispatch_counters(pmc(PASS_B, "pmcW", drv + ["--steps", str(args.steps), "--skip", masks]))
    copy_cmd = [BENCH, "--copy-mib", "256", "--steps", "5"]
    cf = copy_dispatch_counters(pmc(["FETCH_SIZE"], "copyF", copy_cmd))
    cw = copy_dispatch_counters(pmc(["WRITE_SIZE"], "copyW", copy_cmd))
    copy_bytes = 256 * 2 ** 20
    fetch_scale = copy_bytes / (sum(c["FETCH_SIZE"] for c in cf[1:]) / len(cf[1:]) * 1024)
    write_scale = copy_bytes / (sum(c["WRITE_SIZE"] for c in cw[1:]) / len(cw[1:]) * 1024)
    log(f"copy calibration: FETCH_SIZE x {fetch_scale:.3f}, WRITE_SIZE x {write_scale:.3f}")

    per_mask = args.steps * M
    skip0 = args.warmup * M
    expect = skip0 + per_mask * len(MASKS)
    if len(pa) != expect or len(pb) != expect:
        raise RuntimeError(f"expected {expect} update-kernel dispatches, got {len(pa)} / {len(pb)}")

    def avg(rows, i, key):   # per update: sum over its microbatch launches, mean over updates
        chunk = rows[skip0 + i * per_mask: skip0 + (i + 1) * per_mask]
        return sum(r.get(key, 0.0) for r in chunk) / args.steps

    table = {}
    for i, (label, mask, base) in enumerate(MASKS):
        fetch = avg(pa, i, "FETCH_SIZE") * 1024 * fetch_scale
        write = avg(pb, i, "WRITE_SIZE") * 1024 * write_scale
        mops = avg(pa, i, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = avg(pa, i, "SQ_VALU_MFMA_BUSY_CYCLES")
        active = avg(pa, i, "GRBM_GUI_ACTIVE")
        table[label] = dict(mask=mask, us=ms[mask] * 1e3, hbm=fetch + write, flop=mops * 512.0,
                         util=busy / (active / 8.0 * 1024.0) if active else 0.0, base=base)

    def phase_line(label, t):
        base = table.get(t["base"]) if t["base"] else None
        if base is None:
            return f"| {label} | 0x{t['mask']:03x} | {t['us']:.1f} | | {t['flop'] / 1e9:.1f} | {t['util'] * 100:.1f}% | " \
                   f"{t['hbm'] / 1e6:.1f} | | |"
        dt = (t["us"] - base["us"]) * 1e-6
        dflop = t["flop"] - base["flop"]
        dbytes = t["hbm"] - base["hbm"]
        rate = ""
        if dt > 0:
            if dflop > 1e9:
                rate = f"{dflop / dt / 1e12:.0f} TFLOP/s ({dflop / dt / BF16_PEAK * 100:.0f}% of bf16)"
            else:
                rate = f"{dbytes / dt / 1e12:.2f} TB/s ({dbytes / dt / HBM_PEAK * 100:.0f}% of HBM)"
        return f"| {label} | 0x{t['mask']:03x} | {t['us']:.1f} | {dt * 1e6:.1f} | {t['flop'] / 1e9:.1f} | " \
               f"{t['util'] * 100:.1f}% | {t['hbm'] / 1e6:.1f} | {dbytes / 1e6:.1f} | {rate} |"

    lines = [f"# moe_step_kernel — per-phase profile, {cfg.name}", "",
             f"Workload: {cfg.tokens} tokens x {M} microbatch(es), d_model={cfg.d_model}, d_ff={cfg.d_ff}, "
             f"E={cfg.n_experts}, top-{cfg.top_k}, {cfg.dtype}; the seeded inputs of the tests "
             f"(`python -m synth.dump --config {cfg.name}`). Grid {grid} workgroups. Kernel sources sha256 "
             f"`{kernel_source_sha256()[:16]}…`. Made by `python -m moe_step_megakernel_amd.profile --config "
             f"{cfg.name}{' --fresh' if args.fresh else ''}{' --defer' if args.defer else ''}` (from /tmp with TMPDIR=/tmp), "
             "which runs:", "",
             "```", "moe_step_bench " + shown(drv[1:]) + f" --steps {args.timing_steps} --skip {masks}",
             shown(kt_cmd),
             "rocprofv3 --pmc " + " ".join(PASS_A) + " -f csv -d <work>/pmcA -o pmc -- moe_step_bench ... --steps "
             f"{args.steps} --skip <masks>",
             "rocprofv3 --pmc WRITE_SIZE -f csv -d <work>/pmcW -o pmc -- moe_step_bench ... (same)",
             "rocprofv3 --pmc FETCH_SIZE | WRITE_SIZE ... -- moe_step_bench --copy-mib 256 --steps 5", "```", "",
             "A launch with mask m skips the phases whose bits are set (bit i = phase i; 0x100 = the dispatch "
             "gather inside route_order; 0x200 = the k-way row sum inside the last phase) and reuses the arena of "
             "the previous full launch.  Times are per update (all microbatch launches) from the uncounted run; "
             + ("every update starts from the initial parameters and zero moments (restored outside its timing), "
                "so every mask sees the routing of the first update; " if args.fresh else "") +
             "a phase's cost is its launch minus the skeleton's.  MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; "
             "MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) over the launch; HBM bytes "
             f"= FETCH_SIZE x {fetch_scale:.3f} + WRITE_SIZE x {write_scale:.3f} KiB (the copy calibration).", "",
             "| phases run | mask | µs per update | phase µs | MFMA GFLOP | MFMA util | HBM MB | phase MB | phase rate |",
             "|---|---|---|---|---|---|---|---|---|"]
    for label, _, _ in MASKS:
        lines.append(phase_line(label, table[label]))
    lines += ["", "Steps inside phases (difference of two masks):", "",
              "| step | µs | HBM MB | rate |", "|---|---|---|---|"]
    diffs = {}
    for label, a, b in DIFFS:
        dt = (table[a]["us"] - table[b]["us"]) * 1e-6
        db = table[a]["hbm"] - table[b]["hbm"]
        rate = f"{db / dt / 1e12:.2f} TB/s ({db / dt / HBM_PEAK * 100:.0f}% of HBM)" if dt > 0 else "n/a"
        diffs[label] = dict(us=dt * 1e6, mb=db / 1e6)
        lines.append(f"| {label} | {dt * 1e6:.1f} | {db / 1e6:.1f} | {rate} |")
    lines.append("")
    with open(os.path.join(args.out, f"moe_step_kernel_{cfg.name}_phases.md"), "w") as fh:
        fh.write("\n".join(lines))

    # kernel trace summary
    kl = [f"# moe_step_kernel — rocprofv3 kernel trace, {cfg.name}", "",
          f"Command (from /tmp with TMPDIR=/tmp; inputs from `python -m synth.dump --config {cfg.name} --out "
          f"{inputs}`):", "", "```", shown(kt_cmd), "```", "",
          "`--stats` summary (all kernels of the run):", "",
          "| kernel | calls | total ns | average ns | min ns | max ns |", "|---|---|---|---|---|---|"]
    for r in stats_rows:
        kl.append(f"| {r.get('Name', '')[:90]} | {r.get('Calls', '')} | {r.get('TotalDurationNs', '')} | "
                  f"{r.get('AverageNs', '')} | {r.get('MinNs', '')} | {r.get('MaxNs', '')} |")
    kl += ["", f"Update-kernel launches: {len(durs)} ({args.warmup * M} warm-up, then {len(timed)} timed); "
               f"timed launches mean {sum(timed) / max(1, len(timed)):.1f} µs, min {min(timed):.1f}, "
               f"max {max(timed):.1f}; per update ({M} launch(es)) "
               f"{sum(timed) / max(1, len(timed)) * M:.1f} µs.",
           f"Uncounted driver timing of the same full updates: {ms[0] * 1e3:.1f} µs per update.", ""]
    with open(os.path.join(args.out, f"moe_step_kernel_{cfg.name}_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(kl))

    full = table["full update"]
    doc = {"kernel": f"moe::moe_step_kernel ({grid} workgroups)", "workload": cfg.name,
           "kernel_source_sha256": kernel_source_sha256(),
           "hbm_bytes_per_launch": full["hbm"] / M, "hbm_bytes_per_update": full["hbm"],
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "command": f"python -m moe_step_megakernel_amd.profile --config {cfg.name}" + (" --fresh" if args.fresh else "")
           + (" --defer" if args.defer else ""),
           "measured": time.strftime("%Y-%m-%d"), "steps_inside_phases": diffs}
    with open(os.path.join(args.out, f"moe_step_kernel_{cfg.name}_hbm_traffic.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
    log(f"wrote {args.out}/moe_step_kernel_{cfg.name}_{{phases.md,kernel_trace.md,hbm_traffic.json}}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
