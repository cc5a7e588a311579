"""Decoding of the per-workgroup phase clocks written with MOE_RUN_TRACE.

Layout: trace[wg][phase][3] = (phase start, barrier arrival, barrier release),
in ticks of the GPU's constant 100 MHz clock.  The last phase has no barrier;
its arrival and release are the kernel's end.
"""
from __future__ import annotations

import numpy as np

PHASE_NAMES = ["route", "order", "ffn1", "ffn2", "combine", "bwd_dH_dW2", "bwd_dW1_dXs", "dx_norm_adamw"]
TICKS_PER_US = 100.0


def decode(trace_words, grid: int, n_phases: int = len(PHASE_NAMES)) -> dict:
    tr = np.asarray(trace_words, dtype=np.int64).reshape(grid, n_phases, 3)
    t0 = tr[:, 0, 0].min()
    rel = (tr - t0) / TICKS_PER_US                     # microseconds since the first start
    release = rel[:, :, 2]
    arrive = rel[:, :, 1]
    start = rel[:, :, 0]
    # wall-clock span of each phase: from the previous release (max over workgroups,
    # i.e. when the last workgroup left the barrier) to this release
    prev = np.concatenate([[0.0], release.max(axis=0)[:-1]])
    span = release.max(axis=0) - prev
    busy = arrive - start                               # per workgroup, per phase
    wait = release - arrive
    total = release[:, -1].max()
    idle_frac = wait[:, :-1].sum(axis=1) / np.maximum(release[:, -1] - start[:, 0], 1e-9)
    return {
        "total_us": float(total),
        "phase_us": {n: float(s) for n, s in zip(PHASE_NAMES, span)},
        "phase_busy_max_us": {n: float(b) for n, b in zip(PHASE_NAMES, busy.max(axis=0))},
        "phase_busy_mean_us": {n: float(b) for n, b in zip(PHASE_NAMES, busy.mean(axis=0))},
        "barrier_idle_frac_mean": float(idle_frac.mean()),
        "barrier_idle_frac_max": float(idle_frac.max()),
    }
