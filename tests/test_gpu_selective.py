"""Selective updates on an MI355X: the router (shared) is clipped and updated
after every microbatch, the experts accumulate over a window of W microbatches
and are updated at its end (Latch pages, "Results", table "Other measured
compiler work": shared weights every microbatch, experts every 16).  Each
microbatch launch goes through moe_step_run_groups and is compared with the
oracle's selective_step from the same starting state, on the GPU's own routing;
gates as in test_gpu_parity."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import GpuRun, compare_update, say

pytestmark = pytest.mark.gpu

F32_TOL = dict(grad_tol=1e-5, weight_tol=1e-5, loss_tol=1e-5)
BF16_TOL = dict(grad_tol=0.08, weight_tol=1e-2, loss_tol=1e-2)


def _run_selective(cfg, inp, window, tol):
    say(f"[gpu] selective {cfg.name} T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} "
        f"E={cfg.n_experts} k={cfg.top_k} {cfg.dtype} window={window}")
    run = GpuRun(cfg, inp)
    L = run.layer
    T, E, k, d = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.d_model
    try:
        for i in range(cfg.microbatches):
            params, m, v = (a.astype(np.float64) for a in run.state())
            grads = L.grads.cpu().numpy().astype(np.float64)
            groups = dict(zero_router=True, apply_router=True, step_router=i + 1,
                          zero_experts=(i % window == 0), apply_experts=(i % window == window - 1),
                          step_experts=i // window + 1)
            x, t = run.microbatch(i)
            dbg = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device=run.dev)}
            dx = torch.empty(T, d, dtype=torch.float32, device=run.dev)
            L.run(x, t, tokens_in_update=T, dx=dx, router_bias=run.bias, debug=dbg, groups=groups)
            L.status()
            torch.cuda.synchronize()
            idx = dbg["topk_idx"].cpu().numpy().astype(np.int64)
            out = dict(loss=float(L.stats[0].item()), grad_norm=float(L.stats[1].item()),
                       clip_coef=float(L.stats[2].item()), grads=L.grads.cpu().numpy(),
                       params=L.params.cpu().numpy(), exp_avg=L.exp_avg.cpu().numpy(),
                       exp_avg_sq=L.exp_avg_sq.cpu().numpy(), dx=[dx.cpu().numpy()])
            xm, tm = inp.microbatch(i)
            ref = oracle.selective_step(xm, tm, params, grads, m, v, step_router=groups["step_router"],
                                        step_experts=groups["step_experts"], d=cfg.d_model, f=cfg.d_ff,
                                        E=cfg.n_experts, top_k=cfg.top_k, tokens_in_update=T,
                                        zero_router=True, zero_experts=groups["zero_experts"],
                                        apply_router=True, apply_experts=groups["apply_experts"], lr=cfg.lr,
                                        beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                                        weight_decay=cfg.weight_decay, clip_norm=cfg.clip_norm,
                                        bias=inp.router_bias, forced_topk=idx)
            say(f"  microbatch {i}: experts {'applied' if groups['apply_experts'] else 'accumulating'}")
            errs, bad = compare_update(cfg, out, ref, **tol)
            assert not bad, f"microbatch {i}: {bad}: {errs}"
            if not groups["apply_experts"]:
                # the experts' weights and moments must not move before the window ends
                nr = cfg.d_model * cfg.n_experts
                assert np.array_equal(out["params"][nr:], params[nr:].astype(np.float32))
                assert np.array_equal(out["exp_avg"][nr:], m[nr:].astype(np.float32))
    finally:
        run.close()


def test_selective_fp32_router_every_microbatch_experts_every_3():
    cfg = synth.small_config("selective_f32", 160, 64, 128, 4, 2, "f32", microbatches=6)
    _run_selective(cfg, synth.make_inputs(cfg, 7), 3, F32_TOL)


def test_selective_bf16_router_every_microbatch_experts_every_4():
    cfg = synth.small_config("selective_bf16", 1024, 256, 384, 16, 2, "bf16", microbatches=8)
    _run_selective(cfg, synth.make_inputs(cfg, 8), 4, BF16_TOL)
