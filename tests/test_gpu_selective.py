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


def _run_selective(cfg, inp, window, tol, defer=False):
    say(f"[gpu] selective {cfg.name} T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} "
        f"E={cfg.n_experts} k={cfg.top_k} {cfg.dtype} window={window} deferred={defer}")
    run = GpuRun(cfg, inp, max_microbatches=window if defer else 0)
    L = run.layer
    T, E, k, d = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.d_model
    nr = cfg.d_model * cfg.n_experts
    ogr = None   # deferred: the oracle's running gradient (the GPU holds the experts' only when applying)
    try:
        for i in range(cfg.microbatches):
            params, m, v = (a.astype(np.float64) for a in run.state())
            grads = L.grads.cpu().numpy().astype(np.float64)
            if defer and ogr is not None:
                grads[nr:] = ogr[nr:]
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
            ogr = np.asarray(ref["grads"], dtype=np.float64)
            if defer and not groups["apply_experts"]:
                # deferred: the experts' gradient is formed in the applying launch;
                # until then the router part, weights, moments, loss and dx are checked
                out = dict(out)
                out["grads"] = out["grads"].copy()
                out["grads"][nr:] = ref["grads"][nr:]
            errs, bad = compare_update(cfg, out, ref, **tol)
            assert not bad, f"microbatch {i}: {bad}: {errs}"
            if not groups["apply_experts"]:
                # the experts' weights and moments must not move before the window ends
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


def test_selective_bf16_experts_every_4_deferred_weight_gradients():
    # the same schedule with the experts' weight gradients deferred to the
    # window's applying launch (four slots)
    cfg = synth.small_config("selective_bf16", 1024, 256, 384, 16, 2, "bf16", microbatches=8)
    _run_selective(cfg, synth.make_inputs(cfg, 8), 4, BF16_TOL, defer=True)


def test_deferred_weight_gradients_add_to_unzeroed_gradients():
    # an update whose first launch does not zero the gradients adds to them:
    # deferred and per-launch handles agree (same inputs, same launches) up to
    # the order of fp32 accumulation
    cfg = synth.small_config("deferred_accumulate", 768, 256, 384, 16, 2, "bf16", microbatches=3)
    inp = synth.make_inputs(cfg, 25)
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[0] = 3.0
    inp.router_bias = bias
    results = []
    for slots in (0, 3):
        run = GpuRun(cfg, inp, wg_per_cu=2, max_microbatches=slots)
        L = run.layer
        try:
            for upd, zero_first in ((1, True), (2, False)):
                for mb in range(cfg.microbatches):
                    x, t = run.microbatch(mb)
                    L.run(x, t, tokens_in_update=cfg.tokens_in_update, step=upd, zero_grad=zero_first and mb == 0,
                          apply=mb == cfg.microbatches - 1, router_bias=run.bias)
            torch.cuda.synchronize()
            L.status()
            results.append([a.cpu().numpy().astype(np.float64) for a in (L.grads, L.params, L.exp_avg, L.exp_avg_sq)])
        finally:
            run.close()
    for name, a, b in zip(("grads", "params", "exp_avg", "exp_avg_sq"), results[0], results[1]):
        err = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
        say(f"  {name}: deferred vs per-launch rel-L2 {err:.2e}")
        assert err < 1e-4, (name, err)
