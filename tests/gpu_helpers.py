"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run
the HIP update through the C ABI, and compare with the FP64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from moe_step_megakernel_amd.layer import MoeLayerStep


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def device_tokens(arr_f32, bits, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr_f32, dtype=np.float32)).to(dev)


def split_params(flat, cfg):
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    flat = np.asarray(flat)
    return {"W_r": flat[:d * E], "W1": flat[d * E:d * E + E * d * f], "W2": flat[d * E + E * d * f:]}


class GpuRun:
    """One layer on cuda:0 with the inputs of ``inp`` (all microbatches)."""

    def __init__(self, cfg: synth.LayerConfig, inp: synth.LayerInputs, *, clip_norm=None, wg_per_cu=0,
                 ready_gemm12=False, cooperative=False, max_tokens=None, stream=None):
        self.ready_gemm12 = ready_gemm12
        self.stream = stream
        self.cooperative = cooperative
        self.dev = torch.device("cuda", 0)
        if max_tokens is None:
            max_tokens = max(1, cfg.tokens)
        self.layer = MoeLayerStep(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, max_tokens, cfg.dtype,
                                  lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, adam_eps=cfg.eps,
                                  weight_decay=cfg.weight_decay,
                                  clip_norm=cfg.clip_norm if clip_norm is None else clip_norm,
                                  wg_per_cu=wg_per_cu)
        self.layer.load_params(torch.from_numpy(inp.flat_params()))
        self.set_inputs(cfg, inp)

    def set_inputs(self, cfg: synth.LayerConfig, inp: synth.LayerInputs):
        """Switches the token inputs (the layer shape must not change); the
        weights and moments stay those on the device."""
        self.cfg, self.inp = cfg, inp
        self.x = device_tokens(inp.x, inp.x_bits, cfg.dtype, self.dev)
        self.t = device_tokens(inp.t, inp.t_bits, cfg.dtype, self.dev)
        self.bias = None if inp.router_bias is None else torch.from_numpy(inp.router_bias).to(self.dev)

    def microbatch(self, i):
        T = self.cfg.tokens
        return self.x[i * T:(i + 1) * T], self.t[i * T:(i + 1) * T]

    def update(self, step, *, want_dx=True, debug=True):
        """Runs one whole update (all microbatches); returns host copies of the outputs."""
        cfg = self.cfg
        T, E, k, d = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.d_model
        outs = {"logits": [], "idx": [], "gate": [], "counts": [], "perm": [], "dx": []}
        for mb in range(cfg.microbatches):
            x, t = self.microbatch(mb)
            dbg = None
            if debug:
                dbg = {"router_logits": torch.empty(T, E, dtype=torch.float32, device=self.dev),
                       "topk_idx": torch.empty(T, k, dtype=torch.int32, device=self.dev),
                       "topk_gate": torch.empty(T, k, dtype=torch.float32, device=self.dev),
                       "expert_counts": torch.empty(E, dtype=torch.int32, device=self.dev),
                       "route_perm": torch.empty(T * k, dtype=torch.int32, device=self.dev)}
            dx = torch.empty(T, d, dtype=torch.float32, device=self.dev) if want_dx else None
            self.layer.run(x, t, tokens_in_update=cfg.tokens_in_update, step=step, zero_grad=(mb == 0),
                           apply=(mb == cfg.microbatches - 1), dx=dx, router_bias=self.bias, debug=dbg,
                           ready_gemm12=self.ready_gemm12, cooperative=self.cooperative, stream=self.stream)
            self.layer.status()
            if debug:
                outs["logits"].append(dbg["router_logits"].cpu().numpy())
                outs["idx"].append(dbg["topk_idx"].cpu().numpy().astype(np.int64))
                outs["gate"].append(dbg["topk_gate"].cpu().numpy())
                outs["counts"].append(dbg["expert_counts"].cpu().numpy().astype(np.int64))
                outs["perm"].append(dbg["route_perm"].cpu().numpy().astype(np.int64))
            if want_dx:
                outs["dx"].append(dx.cpu().numpy())
        torch.cuda.synchronize()
        L = self.layer
        outs.update(loss=float(L.stats[0].item()), grad_norm=float(L.stats[1].item()),
                    clip_coef=float(L.stats[2].item()), grads=L.grads.cpu().numpy(), params=L.params.cpu().numpy(),
                    exp_avg=L.exp_avg.cpu().numpy(), exp_avg_sq=L.exp_avg_sq.cpu().numpy())
        return outs

    def state(self):
        L = self.layer
        return L.params.cpu().numpy(), L.exp_avg.cpu().numpy(), L.exp_avg_sq.cpu().numpy()

    def close(self):
        self.layer.close()


def oracle_update(cfg, inp, params, m, v, step, forced_idx, *, clip_norm=None):
    xs = [inp.microbatch(i)[0] for i in range(cfg.microbatches)]
    ts = [inp.microbatch(i)[1] for i in range(cfg.microbatches)]
    return oracle.step(xs, ts, params, m, v, step, d=cfg.d_model, f=cfg.d_ff, E=cfg.n_experts, top_k=cfg.top_k,
                       lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay,
                       clip_norm=cfg.clip_norm if clip_norm is None else clip_norm, bias=inp.router_bias,
                       forced_topk=forced_idx)


def compare_update(cfg, gpu, ref, *, grad_tol, weight_tol, loss_tol, dx=True):
    """Relative-L2 gates per tensor; returns the dict of errors."""
    errs = {"loss": abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"])}
    g_gpu, g_ref = split_params(gpu["grads"], cfg), split_params(ref["grads"], cfg)
    for name in ("W_r", "W1", "W2"):
        errs["d" + name] = rel_l2(g_gpu[name], g_ref[name])
    if dx:
        gdx = np.concatenate(gpu["dx"])
        rdx = np.concatenate(ref["dx"]) if isinstance(ref["dx"], list) else ref["dx"]
        errs["dx"] = rel_l2(gdx, rdx)
    for key in ("params", "exp_avg", "exp_avg_sq"):
        a, b = split_params(gpu[key], cfg), split_params(ref[key], cfg)
        for name in ("W_r", "W1", "W2"):
            errs[f"{key}.{name}"] = rel_l2(a[name], b[name])
    errs["grad_norm"] = abs(gpu["grad_norm"] - ref["grad_norm"]) / ref["grad_norm"]
    errs["clip_coef"] = abs(gpu["clip_coef"] - ref["clip_coef"]) / ref["clip_coef"]
    say(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = []
    if errs["loss"] > loss_tol:
        bad.append("loss")
    for key in ("dW_r", "dW1", "dW2", "dx", "grad_norm"):
        if key in errs and errs[key] > grad_tol:
            bad.append(key)
    for key, val in errs.items():
        if key.startswith(("params.", "exp_avg", "clip_coef")) and val > weight_tol:
            bad.append(key)
    return errs, bad
