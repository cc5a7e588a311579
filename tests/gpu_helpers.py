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
                 ready_gemm12=False, cooperative=False, max_tokens=None, stream=None, memory_rules=0,
                 max_microbatches=0):
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
                                  wg_per_cu=wg_per_cu, memory_rules=memory_rules,
                                  max_microbatches=max_microbatches)
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


TILE = 128   # the kernel's output tile edge (rows and columns of every expert product)


def _tiles2d(a, b):
    """128 x 128 tiles of two [M, N] arrays (ragged edges included)."""
    M, N = a.shape
    for m0 in range(0, M, TILE):
        for n0 in range(0, N, TILE):
            yield f"[{m0}:{min(M, m0 + TILE)},{n0}:{min(N, n0 + TILE)}]", a[m0:m0 + TILE, n0:n0 + TILE], \
                b[m0:m0 + TILE, n0:n0 + TILE]


def local_pieces(name, a, b, cfg):
    """The local units a gate is applied to besides the whole tensor: per expert
    slice for every parameter-shaped tensor (a router column of W_r), per 128 x
    128 tile of each expert's weight gradient, per 128-token block of dx."""
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    base = name.split(".")[-1].lstrip("d") if name != "dx" else "dx"
    grad = name.startswith("d") and name != "dx"
    if name == "dx":
        a2, b2 = a.reshape(-1, d), b.reshape(-1, d)
        for t0 in range(0, a2.shape[0], TILE):
            yield f"tokens[{t0}:{min(a2.shape[0], t0 + TILE)}]", a2[t0:t0 + TILE], b2[t0:t0 + TILE]
        return
    if base == "W_r":
        a2, b2 = a.reshape(d, E), b.reshape(d, E)
        for e in range(E):
            yield f"expert {e}", a2[:, e], b2[:, e]
        return
    shape = (E, d, f) if base == "W1" else (E, f, d)
    a3, b3 = a.reshape(shape), b.reshape(shape)
    for e in range(E):
        yield f"expert {e}", a3[e], b3[e]
        if grad:
            for lab, ta, tb in _tiles2d(a3[e], b3[e]):
                yield f"expert {e} tile {lab}", ta, tb


def max_elem_over_rms(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    m = float(np.max(np.abs(a - b))) if b.size else 0.0
    return m / rms if rms > 0 else m


def compare_update(cfg, gpu, ref, *, grad_tol, weight_tol, loss_tol, dx=True, prev=None):
    """Parity gates of one update against the oracle; returns (errors, failures).

    * Gradients and dx: relative L2 <= grad_tol per tensor and per local piece
      (expert slice, 128 x 128 tile of each expert's weight gradient, 128-token
      block of dx).
    * Weights and both moments: relative L2 <= weight_tol per tensor.  Per
      piece the moments get the bound the gradient gate implies, since with the
      same starting state m is linear and v quadratic in the gradient: m <=
      grad_tol, v <= (1 + grad_tol)^2 - 1.
    * With ``prev`` = (params, exp_avg, exp_avg_sq, step, clip_norm) of the
      state before the update, the optimizer is checked on its own, per tensor
      and per piece: the GPU's W step, m and v against the oracle's AdamW applied
      to the GPU's own pre-clip gradients and clip coefficient, where only fp32
      rounding separates the two (1e-4, plus one fp32 rounding of the stored
      weight for the step); and the GPU's step W - W_prev against the oracle's
      per tensor, at the bound the gradient gate implies once AdamW's first
      steps turn gradient errors into sign flips (a flip fraction of about e/pi
      for a relative gradient error e, each flip a step error of two lr: a step
      relative L2 of 2 sqrt(e/pi))."""
    errs = {"loss": abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"])}
    worst, maxrel, bad = {}, {}, []
    m_tol, v_tol = grad_tol, (1.0 + grad_tol) ** 2 - 1.0
    tensors = []
    g_gpu, g_ref = split_params(gpu["grads"], cfg), split_params(ref["grads"], cfg)
    for name in ("W_r", "W1", "W2"):
        tensors.append(("d" + name, g_gpu[name], g_ref[name], grad_tol, grad_tol))
    if dx:
        gdx = np.concatenate(gpu["dx"])
        rdx = np.concatenate(ref["dx"]) if isinstance(ref["dx"], list) else ref["dx"]
        tensors.append(("dx", gdx, rdx, grad_tol, grad_tol))
    for key, ptol in (("params", None), ("exp_avg", m_tol), ("exp_avg_sq", v_tol)):
        a, b = split_params(gpu[key], cfg), split_params(ref[key], cfg)
        for name in ("W_r", "W1", "W2"):
            tensors.append((f"{key}.{name}", a[name], b[name], weight_tol, ptol))
    for name, a, b, tol, ptol in tensors:
        errs[name] = rel_l2(a, b)
        if errs[name] > tol:
            bad.append(name)
        maxrel[name] = max_elem_over_rms(a, b)
        if ptol is None:
            continue
        wl, wv = None, -1.0
        for lab, pa, pb in local_pieces(name, a, b, cfg):
            e = rel_l2(pa, pb)
            if e > wv:
                wl, wv = lab, e
            if e > ptol:
                bad.append(f"{name} {lab} ({e:.3g})")
        if wl is not None:
            worst[name] = (wl, wv)
    errs["grad_norm"] = abs(gpu["grad_norm"] - ref["grad_norm"]) / ref["grad_norm"]
    errs["clip_coef"] = abs(gpu["clip_coef"] - ref["clip_coef"]) / ref["clip_coef"]
    if errs["loss"] > loss_tol:
        bad.append("loss")
    if errs["grad_norm"] > grad_tol:
        bad.append("grad_norm")
    if errs["clip_coef"] > weight_tol:
        bad.append("clip_coef")
    if prev is not None:
        bad += _check_optimizer(cfg, gpu, ref, prev, grad_tol, errs, worst)
    say(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    say("  worst local piece: " + "; ".join(f"{k} {lab} {v:.2e}" for k, (lab, v) in worst.items()))
    say("  max element error / RMS: " + " ".join(f"{k}={v:.2e}" for k, v in maxrel.items()))
    return errs, bad


def step_error(new_gpu, new_ref, old, tol):
    """Relative L2 error of a weight step (new - old) and whether it is within
    tol.  The stored weight is fp32, so the step of each element is only known
    to one rounding of the new weight (2^-24 of it, 2^-23 allowed): for a step
    far smaller than the weight (pure decay, lr * wd * w) that rounding, not the
    arithmetic, sets the error, and the bound adds it."""
    a = np.asarray(new_gpu, np.float64) - old
    b = np.asarray(new_ref, np.float64) - old
    err = float(np.linalg.norm(a - b))
    nb = float(np.linalg.norm(b))
    bound = tol * nb + 2.0 ** -23 * float(np.linalg.norm(np.asarray(new_ref, np.float64)))
    return (err / nb if nb > 0 else err), err <= bound


def _check_optimizer(cfg, gpu, ref, prev, grad_tol, errs, worst):
    p0, m0, v0, step, clip_norm = prev
    bad = []
    step_tol = 2.0 * np.sqrt(grad_tol / np.pi)
    wg, wr, w0 = split_params(gpu["params"], cfg), split_params(ref["params"], cfg), split_params(p0, cfg)
    for name in ("W_r", "W1", "W2"):
        e, ok = step_error(wg[name], wr[name], w0[name], step_tol)
        errs[f"step.{name}"] = e
        if not ok:
            bad.append(f"step.{name}")
    # AdamW on the GPU's own gradients: isolates the optimizer arithmetic
    g = np.asarray(gpu["grads"], np.float64)
    c_own = oracle.clip_coefficient(oracle.global_norm([g]), clip_norm)
    errs["clip_vs_own_norm"] = abs(gpu["clip_coef"] - c_own) / c_own
    if errs["clip_vs_own_norm"] > 1e-5:
        bad.append("clip_vs_own_norm")
    w1, m1, v1 = oracle.adamw(p0, gpu["clip_coef"] * g, m0, v0, step, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps,
                              cfg.weight_decay)
    for key, mine, own, old in (("params", gpu["params"], w1, p0), ("exp_avg", gpu["exp_avg"], m1, None),
                                ("exp_avg_sq", gpu["exp_avg_sq"], v1, None)):
        a, b = split_params(mine, cfg), split_params(own, cfg)
        o = split_params(np.asarray(old, np.float64), cfg) if old is not None else None
        for name in ("W_r", "W1", "W2"):
            tag = f"adamw_own.{key}.{name}"
            wl, wv = None, -1.0
            whole = [("", a[name], b[name])]
            parts = list(local_pieces(f"{key}.{name}", a[name], b[name], cfg))
            opar = list(local_pieces(f"{key}.{name}", o[name], o[name], cfg)) if o is not None else None
            for i, (lab, pa, pb) in enumerate(whole + parts):
                po = None if o is None else (o[name] if i == 0 else opar[i - 1][1])
                if po is not None:   # the step itself, not the weights it is added to
                    e, ok = step_error(pa, pb, po, 1e-4)
                else:
                    e = rel_l2(pa, pb)
                    ok = e <= 1e-4
                if i == 0:
                    errs[tag] = e
                elif e > wv:
                    wl, wv = lab, e
                if not ok:
                    bad.append(f"{tag} {lab}".rstrip() + f" ({e:.3g})")
            if wl is not None:
                worst[tag] = (wl, wv)
    return bad
