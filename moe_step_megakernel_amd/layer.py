"""Training state of one MoE feed-forward layer on the GPU, driven through the
C ABI.  Holds the caller-owned tensors (fp32 master weights, gradients, Adam
moments, stats) and hands their pointers to ``moe_step_run``; it computes
nothing itself."""
from __future__ import annotations

import torch

from . import binding as B


class MoeLayerStep:
    def __init__(self, d_model, d_ff, n_experts, top_k, max_tokens, dtype="bf16", lr=1e-3, beta1=0.9,
                 beta2=0.999, adam_eps=1e-8, weight_decay=0.01, clip_norm=1.0, device=0, wg_per_cu=0,
                 memory_rules=0, max_microbatches=0):
        self.cfg = B.make_config(d_model, d_ff, n_experts, top_k, max_tokens, dtype, lr, beta1, beta2, adam_eps,
                                 weight_decay, clip_norm, device, wg_per_cu, memory_rules, max_microbatches)
        self.dtype = dtype
        self.dev = torch.device("cuda", device)
        self.P = B.moe_step_param_count(self.cfg)
        self.handle = B.moe_step_create(self.cfg)
        self.grid = B.moe_step_grid_size(self.handle)
        z = lambda: torch.zeros(self.P, dtype=torch.float32, device=self.dev)  # noqa: E731
        self.params, self.grads, self.exp_avg, self.exp_avg_sq = z(), z(), z(), z()
        self.stats = torch.zeros(4, dtype=torch.float32, device=self.dev)
        self._shadow_valid = False

    def load_params(self, flat):
        """Copies fp32 master weights in (W_r | W1 | W2 order); resets the moments."""
        self.params.copy_(torch.as_tensor(flat, dtype=torch.float32))
        self.exp_avg.zero_()
        self.exp_avg_sq.zero_()
        self._shadow_valid = False

    def run(self, x, target, *, tokens_in_update=None, step=1, zero_grad=True, apply=True, dx=None,
            router_bias=None, debug=None, trace=None, stream=None, groups=None, ready_gemm12=False,
            cooperative=False, refresh_shadow=False, test_timeout=False, barrier_per_workgroup=False):
        """Enqueues one launch.  ``debug`` is an optional dict of preallocated debug tensors
        (router_logits, topk_idx, topk_gate, expert_counts, route_perm).  ``groups`` (selective
        updates) replaces zero_grad/apply/step by per-group settings: a dict with keys
        zero_router, zero_experts, apply_router, apply_experts (bools) and step_router,
        step_experts (ints).  ``ready_gemm12`` replaces the grid barrier between the two
        expert products by per-row-tile readiness counters (same results).  ``cooperative``
        launches through hipLaunchCooperativeKernel instead of an ordinary launch.
        ``refresh_shadow`` rebuilds the bf16 weight copy from params even when it is
        current; ``test_timeout`` sets the failure-path test flag (the launch ends
        with a grid-barrier timeout); ``barrier_per_workgroup`` makes every workgroup write its
        XCD's L2 back at each grid barrier instead of one workgroup per XCD (same results)."""
        n = 0 if x is None else int(x.shape[0])
        self._check_tensors(n, x, target, dx, router_bias, debug or {}, trace)
        flags = 0
        step_r = step_e = step
        if groups is not None:
            for key, bit in (("zero_router", B.MOE_RUN_ZERO_GRAD_ROUTER), ("zero_experts", B.MOE_RUN_ZERO_GRAD_EXPERTS),
                             ("apply_router", B.MOE_RUN_APPLY_ROUTER), ("apply_experts", B.MOE_RUN_APPLY_EXPERTS)):
                if groups.get(key):
                    flags |= bit
            step_r, step_e = int(groups.get("step_router", 1)), int(groups.get("step_experts", 1))
        else:
            if zero_grad:
                flags |= B.MOE_RUN_ZERO_GRAD
            if apply:
                flags |= B.MOE_RUN_APPLY
        if refresh_shadow or not self._shadow_valid:
            flags |= B.MOE_RUN_REFRESH_SHADOW
        if test_timeout:
            flags |= B.MOE_RUN_TEST_TIMEOUT
        if barrier_per_workgroup:
            flags |= B.MOE_RUN_BARRIER_PER_WORKGROUP
        if trace is not None:
            flags |= B.MOE_RUN_TRACE
        if ready_gemm12:
            flags |= B.MOE_RUN_READY_GEMM12
        if cooperative:
            flags |= B.MOE_RUN_COOPERATIVE
        dbg = debug or {}
        io = B.make_io(x=x, target=target, router_bias=router_bias, params=self.params, grads=self.grads,
                       exp_avg=self.exp_avg, exp_avg_sq=self.exp_avg_sq, dx=dx, stats=self.stats,
                       router_logits=dbg.get("router_logits"), topk_idx=dbg.get("topk_idx"),
                       topk_gate=dbg.get("topk_gate"), expert_counts=dbg.get("expert_counts"),
                       route_perm=dbg.get("route_perm"), trace=trace)
        s = torch.cuda.current_stream(self.dev) if stream is None else stream
        B.moe_step_run_groups(self.handle, io, n, tokens_in_update or max(1, n), step_r, step_e, flags,
                              s.cuda_stream)
        self._shadow_valid = True

    def _check_tensors(self, n, x, target, dx, router_bias, debug, trace):
        """The C ABI takes bare device pointers, so every tensor is checked here
        (device, dtype, contiguity, shape) before its pointer goes to the kernel."""
        d, E, k = self.cfg.d_model, self.cfg.n_experts, self.cfg.top_k
        act = torch.bfloat16 if self.dtype == "bf16" else torch.float32

        def check(name, t, dtype, shape):
            if t is None:
                return
            if not isinstance(t, torch.Tensor) or t.device != self.dev:
                raise ValueError(f"{name} must be a tensor on {self.dev}")
            if t.dtype != dtype:
                raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")

        if (x is None) != (target is None):
            raise ValueError("x and target are given together or not at all")
        check("x", x, act, (n, d))
        check("target", target, act, (n, d))
        check("dx", dx, torch.float32, (n, d))
        check("router_bias", router_bias, torch.float32, (E,))
        shapes = {"router_logits": (torch.float32, (n, E)), "topk_idx": (torch.int32, (n, k)),
                  "topk_gate": (torch.float32, (n, k)), "expert_counts": (torch.int32, (E,)),
                  "route_perm": (torch.int32, (n * k,))}
        for name, t in debug.items():
            if name not in shapes:
                raise ValueError(f"unknown debug output {name}")
            check(name, t, *shapes[name])
        if trace is not None:
            check("trace", trace, torch.int64, tuple(trace.shape))
            if trace.numel() < self.trace_words():
                raise ValueError(f"trace needs {self.trace_words()} words, got {trace.numel()}")

    def status(self):
        B.moe_step_status(self.handle)

    def check_guards(self):
        """Raises MoeStepError unless every guard zone of the arena is intact
        (handles made with memory_rules including MOE_MEM_GUARDS)."""
        B.moe_step_check_guards(self.handle)

    def trace_words(self):
        return B.moe_step_trace_words(self.handle)

    def arena_bytes(self):
        return B.moe_step_arena_bytes(self.handle)

    def close(self):
        if self.handle:
            B.moe_step_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
