"""Parity of the HIP update with the FP64 oracle on an MI355X.

Routing (top-k indices, expert counts, route_order permutation) must be bit-exact
given the GPU's own fp32 router logits.  Floating-point outputs are compared per
tensor with relative L2:
  fp32 mode: every output <= 1e-5;
  bf16 mode: gradients and dx <= 0.08 (the pages' FP64 gradient gate, Latch
  "Results", numerical scope), updated weights and moments <= 1e-2, loss <= 1e-2.
The full-step oracle runs with the GPU's selection (``forced_topk``) so a near-tie
that fp32 and fp64 logits resolve differently cannot fail a numeric gate; the
number of tokens whose FP64 routing differs is printed."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import GpuRun, compare_update, oracle_update, rel_l2, say
from moe_step_megakernel_amd import binding as B

pytestmark = pytest.mark.gpu

F32_TOL = dict(grad_tol=1e-5, weight_tol=1e-5, loss_tol=1e-5)
BF16_TOL = dict(grad_tol=0.08, weight_tol=1e-2, loss_tol=1e-2)


def _check_routing(cfg, inp, out, w_router):
    for mb in range(cfg.microbatches):
        z = out["logits"][mb].astype(np.float64)
        ref_idx = oracle.token_topk(z, cfg.top_k)
        np.testing.assert_array_equal(out["idx"][mb], ref_idx)
        counts, offsets, perm, inv = oracle.route_order(ref_idx, cfg.n_experts)
        np.testing.assert_array_equal(out["counts"][mb], counts)
        np.testing.assert_array_equal(out["perm"][mb], perm)
        np.testing.assert_allclose(out["gate"][mb], oracle.topk_gates(z, ref_idx), rtol=2e-6, atol=1e-7)
        x, _ = inp.microbatch(mb)
        zr = oracle.router_logits(x, w_router, inp.router_bias)
        assert rel_l2(z, zr) < 1e-5
        diff = int((oracle.token_topk(zr, cfg.top_k) != ref_idx).any(axis=1).sum())
        if mb == 0 or mb == cfg.microbatches - 1:
            say(f"  microbatch {mb}: tokens routed differently by FP64 logits: {diff}; "
                f"rows per expert min {counts.min()} max {counts.max()}")


def _run_and_compare(cfg, inp, tol, *, steps=2, clip_norm=None, wg_per_cu=0, ready_gemm12=False, cooperative=False,
                     memory_rules=0, max_microbatches=0):
    say(f"[gpu] {cfg.name} T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} E={cfg.n_experts} "
        f"k={cfg.top_k} {cfg.dtype} clip={cfg.clip_norm if clip_norm is None else clip_norm} "
        f"wg_per_cu={wg_per_cu} memory_rules={memory_rules} max_microbatches={max_microbatches}")
    run = GpuRun(cfg, inp, clip_norm=clip_norm, wg_per_cu=wg_per_cu, ready_gemm12=ready_gemm12,
                 cooperative=cooperative, memory_rules=memory_rules, max_microbatches=max_microbatches)
    try:
        params = inp.flat_params().astype(np.float64)
        m = np.zeros_like(params)
        v = np.zeros_like(params)
        for s in range(1, steps + 1):
            out = run.update(s)
            _check_routing(cfg, inp, out, params[:cfg.d_model * cfg.n_experts].reshape(cfg.d_model, cfg.n_experts))
            ref = oracle_update(cfg, inp, params, m, v, s, out["idx"], clip_norm=clip_norm)
            errs, bad = compare_update(cfg, out, ref, **tol,
                                       prev=(params, m, v, s, cfg.clip_norm if clip_norm is None else clip_norm))
            assert not bad, f"step {s}: {bad}: {errs}"
            # the next step starts from the GPU's state so each step is checked on its own
            params, m, v = (a.astype(np.float64) for a in run.state())
    finally:
        run.close()


def test_tiny_f32_two_steps():
    cfg = synth.CONFIGS["tiny_f32"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), F32_TOL)


def test_tiny_f32_clipping_active():
    cfg = synth.CONFIGS["tiny_f32"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), F32_TOL, steps=1, clip_norm=0.1)


@pytest.mark.parametrize("T,d,f,E,k", [(333, 72, 136, 5, 2), (77, 8, 8, 1, 1), (190, 64, 200, 7, 7),
                                       (257, 136, 264, 64, 8)])
def test_ragged_shapes_f32(T, d, f, E, k):
    cfg = synth.small_config("ragged_f32", T, d, f, E, k, "f32")
    _run_and_compare(cfg, synth.make_inputs(cfg, 3), F32_TOL, steps=1)


@pytest.mark.parametrize("T,d,f,E,k", [(333, 72, 136, 5, 2), (1000, 256, 384, 16, 2), (300, 128, 64, 64, 8)])
def test_ragged_shapes_bf16(T, d, f, E, k):
    cfg = synth.small_config("ragged_bf16", T, d, f, E, k, "bf16")
    _run_and_compare(cfg, synth.make_inputs(cfg, 4), BF16_TOL, steps=1)


@pytest.mark.parametrize("T,d,f,E,k", [(333, 72, 136, 5, 2), (1000, 256, 384, 16, 2), (300, 128, 64, 64, 8)])
def test_ragged_shapes_bf16_two_workgroups_per_cu(T, d, f, E, k):
    # the kernel built for two workgroups per compute unit: 2-stage GEMM
    # pipeline, half the LDS, router passes of 16 experts (E = 64 takes four)
    cfg = synth.small_config("ragged_bf16_occ2", T, d, f, E, k, "bf16")
    _run_and_compare(cfg, synth.make_inputs(cfg, 4), BF16_TOL, steps=1, wg_per_cu=2)


@pytest.mark.parametrize("dtype,T,d,f,E,k,wg_per_cu", [("f32", 1, 8, 8, 3, 2, 1), ("bf16", 1, 8, 8, 3, 2, 1),
                                                       ("bf16", 1, 8, 8, 3, 2, 2), ("bf16", 5, 16, 24, 2, 1, 1),
                                                       ("f32", 5, 16, 24, 2, 1, 1)])
def test_minimum_shapes(dtype, T, d, f, E, k, wg_per_cu):
    # the smallest sizes the boundary accepts: one token, d = f = 8 (a single
    # valid 8-element piece in every 64-deep k-tile and 128-wide column tile)
    cfg = synth.small_config(f"minimum_{dtype}_T{T}", T, d, f, E, k, dtype)
    _run_and_compare(cfg, synth.make_inputs(cfg, 9), BF16_TOL if dtype == "bf16" else F32_TOL, steps=2,
                     wg_per_cu=wg_per_cu)


@pytest.mark.parametrize("dtype,E,k,wg_per_cu", [("f32", 1, 1, 1), ("bf16", 1, 1, 1), ("bf16", 1, 1, 2),
                                                ("bf16", 2, 2, 1)])
def test_degenerate_expert_counts(dtype, E, k, wg_per_cu):
    # one expert (every token routed to it with gate 1, the router gradient
    # is zero) and top-k = E (every expert chosen by every token)
    cfg = synth.small_config(f"degenerate_{dtype}_E{E}k{k}", 997, 96, 64, E, k, dtype)
    _run_and_compare(cfg, synth.make_inputs(cfg, 8), BF16_TOL if dtype == "bf16" else F32_TOL, steps=2,
                     wg_per_cu=wg_per_cu)


@pytest.mark.parametrize("dtype,wg_per_cu,T", [("bf16", 1, 16 * 256 + 352), ("bf16", 2, 16 * 512 + 704),
                                              ("f32", 1, 16 * 256 + 352)])
def test_router_several_tokens_per_lane(dtype, wg_per_cu, T):
    # 17 tokens per workgroup: the router pass covers 32 token slots with
    # several tokens per lane, and the last lane group holds one live token
    cfg = synth.small_config(f"router_tl_{dtype}", T, 96, 64, 12, 2, dtype)
    _run_and_compare(cfg, synth.make_inputs(cfg, 6), BF16_TOL if dtype == "bf16" else F32_TOL, steps=1,
                     wg_per_cu=wg_per_cu)


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_readiness_counters_between_expert_products(wg_per_cu):
    # no grid barrier between GEMM 1 and GEMM 2: per-row-tile ready counters
    # (both kernels; the fp32 path and a ragged bf16 shape with E = 64)
    for cfg, seed, tol in ((synth.small_config("ready_f32", 333, 72, 136, 5, 2, "f32"), 3, F32_TOL),
                           (synth.small_config("ready_bf16", 300, 128, 64, 64, 8, "bf16"), 4, BF16_TOL),
                           (synth.CONFIGS["bf16_2x1024"], 0, BF16_TOL)):
        _run_and_compare(cfg, synth.make_inputs(cfg, seed), tol, steps=1, wg_per_cu=wg_per_cu, ready_gemm12=True)


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_cooperative_launch(wg_per_cu):
    # the same kernel through hipLaunchCooperativeKernel
    for cfg, seed, tol in ((synth.CONFIGS["tiny_f32"], 0, F32_TOL), (synth.CONFIGS["bf16_2x1024"], 0, BF16_TOL)):
        _run_and_compare(cfg, synth.make_inputs(cfg, seed), tol, steps=1, wg_per_cu=wg_per_cu, cooperative=True)


def test_bf16_2x1024_two_steps():
    cfg = synth.CONFIGS["bf16_2x1024"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL)


def test_bf16_2x1024_one_workgroup_per_cu():
    # the 2x1024 workload on the kernel built for one workgroup per CU (the
    # automatic choice there is two)
    cfg = synth.CONFIGS["bf16_2x1024"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL, steps=1, wg_per_cu=1)


def test_routing_ties_and_empty_experts():
    # identical router columns give bitwise-identical logits: the lower expert index
    # must win; a zero router sends every token to experts 0..k-1 (the rest get no rows)
    cfg = synth.small_config("ties", 200, 64, 64, 6, 2, "f32")
    inp = synth.make_inputs(cfg, 5)
    inp.w_router[:, 3] = inp.w_router[:, 1]
    inp.w_router[:, 5] = inp.w_router[:, 0]
    _run_and_compare(cfg, inp, F32_TOL, steps=1)
    inp.w_router[:] = 0.0
    run = GpuRun(cfg, inp)
    try:
        out = run.update(1)
        assert np.all(out["idx"][0] == np.array([0, 1]))
        np.testing.assert_array_equal(out["counts"][0], [200, 200, 0, 0, 0, 0])
        np.testing.assert_allclose(out["gate"][0], 0.5, rtol=0, atol=0)
    finally:
        run.close()


@pytest.mark.parametrize("dtype,T,d,f,E,mb,wg_per_cu", [("f32", 300, 72, 136, 5, 3, 1),
                                                        ("bf16", 1000, 256, 384, 16, 2, 1),
                                                        ("bf16", 1000, 256, 384, 16, 2, 2)])
def test_skewed_routing_split_contractions(dtype, T, d, f, E, mb, wg_per_cu):
    # a router bias sends most tokens to experts 0 and 1: their weight-gradient
    # contractions are split into chunks, the partial tiles added back in the
    # following phase (and the one after it), over accumulated microbatches
    cfg = synth.small_config("skewed", T, d, f, E, 2, dtype, microbatches=mb)
    inp = synth.make_inputs(cfg, 8)
    bias = np.zeros(E, np.float32)
    bias[0], bias[1] = 4.0, 2.0
    inp.router_bias = bias
    _run_and_compare(cfg, inp, F32_TOL if dtype == "f32" else BF16_TOL, steps=1, wg_per_cu=wg_per_cu)


def test_f32_at_the_layer_shape():
    # fp32 mode at the bf16 workloads' layer shape (d = 768, f = 1536, 16
    # experts, top-2, 2048 tokens): contractions of 768 and 1536 terms and
    # about 256 routed rows per expert, still within 1e-5 over two updates
    cfg = synth.small_config("f32_2x1024_shape", 2048, 768, 1536, 16, 2, "f32")
    _run_and_compare(cfg, synth.make_inputs(cfg, 13), F32_TOL, steps=2)


@pytest.mark.timeout(900)
def test_max_tokens_limit():
    # the most tokens a handle accepts (2^24, with narrow d = f = 8 so the
    # arena stays near 4 GB): 32,768 tokens per workgroup in routing and
    # route_order, a weight-gradient contraction over about 8.4 M rows per
    # expert, 131,072 router-gradient chunks; one update against the oracle
    cfg = synth.small_config("max_tokens_bf16", 1 << 24, 8, 8, 4, 2, "bf16")
    _run_and_compare(cfg, synth.make_inputs(cfg, 14), BF16_TOL, steps=1)


def test_gradient_accumulation_f32():
    cfg = synth.small_config("accum_f32", 96, 64, 128, 4, 2, "f32", microbatches=3)
    _run_and_compare(cfg, synth.make_inputs(cfg, 6), F32_TOL, steps=1)


def test_deterministic_reruns():
    cfg = synth.CONFIGS["bf16_2x1024"]
    inp = synth.make_inputs(cfg, 1)
    outs = []
    for _ in range(2):
        run = GpuRun(cfg, inp)
        try:
            outs.append(run.update(1))
        finally:
            run.close()
    for key in ("grads", "params", "exp_avg", "exp_avg_sq"):
        assert np.array_equal(outs[0][key], outs[1][key]), key
    assert np.array_equal(outs[0]["dx"][0], outs[1]["dx"][0])
    assert outs[0]["loss"] == outs[1]["loss"]


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_side_stream_matches_default_stream(wg_per_cu):
    # the update enqueued on a caller's stream instead of the default one: same
    # bits (the update is deterministic), and the oracle gates on the first run
    cfg = synth.small_config("side_stream_bf16", 1000, 256, 384, 16, 2, "bf16")
    inp = synth.make_inputs(cfg, 12)
    side = torch.cuda.Stream(device=0)
    outs = []
    for stream in (None, side):
        run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu, stream=stream)
        try:
            torch.cuda.synchronize()   # inputs and weights were copied on the default stream
            outs.append(run.update(1))
        finally:
            run.close()
    params = inp.flat_params().astype(np.float64)
    ref = oracle_update(cfg, inp, params, np.zeros_like(params), np.zeros_like(params), 1, outs[1]["idx"])
    errs, bad = compare_update(cfg, outs[1], ref, **BF16_TOL)
    assert not bad, f"side stream: {bad}: {errs}"
    for key in ("grads", "params", "exp_avg", "exp_avg_sq"):
        assert np.array_equal(outs[0][key], outs[1][key]), key
    assert np.array_equal(outs[0]["dx"][0], outs[1]["dx"][0])
    assert outs[0]["loss"] == outs[1]["loss"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_logit_reported_and_handle_recovers(dtype):
    # a NaN in one token's activations makes its router logits NaN: the kernel
    # flags it (every index it derives stays in range), moe_step_status reports
    # it, and after that the same handle runs a clean update that matches
    cfg = synth.small_config(f"nonfinite_{dtype}", 96, 64, 128, 4, 2, dtype)
    inp = synth.make_inputs(cfg, 15)
    run = GpuRun(cfg, inp)
    try:
        x = run.x.clone()
        x[5, 3] = float("nan")
        run.layer.run(x, run.t, step=1)
        with pytest.raises(B.MoeStepError) as ei:
            run.layer.status()
        assert ei.value.status == B.MOE_ERR_DEVICE
        assert "non-finite router logit" in str(ei.value)
        run.layer.load_params(torch.from_numpy(inp.flat_params()))
        out = run.update(1)
        params = inp.flat_params().astype(np.float64)
        ref = oracle_update(cfg, inp, params, np.zeros_like(params), np.zeros_like(params), 1, out["idx"])
        errs, bad = compare_update(cfg, out, ref, **(BF16_TOL if dtype == "bf16" else F32_TOL))
        assert not bad, f"update after the reported error: {bad}: {errs}"
    finally:
        run.close()


def test_zero_tokens_only_decays():
    cfg = synth.small_config("empty", 0, 64, 128, 4, 2, "f32")
    inp = synth.make_inputs(synth.small_config("empty_src", 1, 64, 128, 4, 2, "f32"), 0)
    run = GpuRun(cfg, inp)
    try:
        p0 = inp.flat_params().astype(np.float64)
        run.layer.run(None, None, tokens_in_update=1, step=1, zero_grad=True, apply=True)
        run.layer.status()
        torch.cuda.synchronize()
        assert np.all(run.layer.grads.cpu().numpy() == 0.0)
        assert rel_l2(run.layer.params.cpu().numpy(), p0 * (1 - cfg.lr * cfg.weight_decay)) < 1e-7
    finally:
        run.close()


@pytest.mark.parametrize("dtype,wg_per_cu,tmax,d,f,E,k,token_counts", [
    ("f32", 1, 1000, 72, 136, 5, 2, (1000, 77, 513, 1)),
    # d = 1024 over 256 workgroups: the router-gradient partials of 8064 and
    # 4032 tokens take 126 chunks (64 and 32 tokens each), more than the 71 of
    # max_tokens = 9000 (chunks of 128)
    ("bf16", 1, 9000, 1024, 64, 16, 2, (9000, 8064, 4032, 333)),
    # over 512 workgroups: 8128 tokens take 254 chunks of 32, 9000 take 141 of 64
    ("bf16", 2, 9000, 1024, 64, 16, 2, (9000, 8128, 1, 2999)),
    ("bf16", 1, 600, 128, 64, 64, 8, (600, 37, 599)),
])
def test_handle_reused_across_token_counts(dtype, wg_per_cu, tmax, d, f, E, k, token_counts):
    # one handle, sized for max_tokens, runs updates of fewer tokens in turn
    # (arena, grid and kernel stay those chosen at create); each update is
    # checked against the oracle from the device state before it
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    cfg0 = synth.small_config(f"reuse_{dtype}", tmax, d, f, E, k, dtype)
    inp0 = synth.make_inputs(cfg0, 11)
    say(f"[gpu] handle reuse {dtype} wg_per_cu={wg_per_cu} max_tokens={tmax} d={d} f={f} E={E} k={k} "
        f"token counts {token_counts}")
    run = GpuRun(cfg0, inp0, wg_per_cu=wg_per_cu, max_tokens=tmax)
    try:
        params = inp0.flat_params().astype(np.float64)
        m = np.zeros_like(params)
        v = np.zeros_like(params)
        for s, T in enumerate(token_counts, start=1):
            cfg = synth.small_config(f"reuse_{dtype}_T{T}", T, d, f, E, k, dtype)
            inp = synth.make_inputs(cfg, 20 + s)
            run.set_inputs(cfg, inp)
            say(f"  update {s}: {T} tokens")
            out = run.update(s)
            _check_routing(cfg, inp, out, params[:d * E].reshape(d, E))
            ref = oracle_update(cfg, inp, params, m, v, s, out["idx"])
            errs, bad = compare_update(cfg, out, ref, **tol, prev=(params, m, v, s, cfg.clip_norm))
            assert not bad, f"update {s} ({T} tokens): {bad}: {errs}"
            params, m, v = (a.astype(np.float64) for a in run.state())
        if dtype == "f32":
            # more tokens than max_tokens: refused on the host, the handle keeps working
            x = torch.zeros(tmax + 1, d, dtype=torch.float32, device=run.dev)
            with pytest.raises(B.MoeStepError):
                run.layer.run(x, x, step=len(token_counts) + 1)
            out = run.update(len(token_counts) + 1)
            ref = oracle_update(run.cfg, run.inp, params, m, v, len(token_counts) + 1, out["idx"])
            errs, bad = compare_update(run.cfg, out, ref, **tol)
            assert not bad, f"update after a refused call: {bad}: {errs}"
    finally:
        run.close()


# ----------------------------------------------------------------------------
# The full-size workloads, in the launch configuration bench.py times
# ----------------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_bf16_32x1024_full_size():
    cfg = synth.CONFIGS["bf16_32x1024"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL, steps=1)


@pytest.mark.timeout(900)
def test_top8_4x1024_full_size():
    cfg = synth.CONFIGS["top8_4x1024"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL, steps=2)


@pytest.mark.parametrize("T,d,f,E,k,mb,wg_per_cu,skew,slots", [
    (1000, 256, 384, 16, 2, 3, 2, True, 3),    # split chunks over the slots' concatenated rows
    (1000, 256, 384, 16, 2, 3, 1, True, 16),   # the one-per-CU kernel, spare slots
    (700, 128, 256, 8, 2, 4, 2, False, 4),     # balanced routing
    (513, 256, 128, 64, 8, 2, 1, False, 2),    # 64 experts, top-8, empty experts in some slots
    (1000, 256, 384, 16, 2, 1, 2, True, 2),    # one microbatch: slot 0 applies
])
def test_deferred_weight_gradients(T, d, f, E, k, mb, wg_per_cu, skew, slots):
    # max_microbatches > 1: each microbatch launch keeps its dW operand rows
    # in a slot and the applying launch contracts dW1 / dW2 over all slots;
    # the same update within the same gates, over two updates (the slots are
    # reused by the second)
    cfg = synth.small_config("deferred", T, d, f, E, k, "bf16", microbatches=mb)
    inp = synth.make_inputs(cfg, 23)
    if skew:
        bias = np.zeros(E, np.float32)
        bias[0], bias[1] = 4.0, 2.0
        inp.router_bias = bias
    _run_and_compare(cfg, inp, BF16_TOL, steps=2, wg_per_cu=wg_per_cu, max_microbatches=slots)


@pytest.mark.parametrize("ready_gemm12,cooperative", [(True, False), (False, True)])
def test_deferred_weight_gradients_other_launch_modes(ready_gemm12, cooperative):
    # deferral with the readiness counters between the expert products, and
    # with a cooperative launch
    cfg = synth.small_config("deferred_modes", 1000, 256, 384, 16, 2, "bf16", microbatches=3)
    inp = synth.make_inputs(cfg, 26)
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[0], bias[1] = 4.0, 2.0
    inp.router_bias = bias
    _run_and_compare(cfg, inp, BF16_TOL, steps=2, wg_per_cu=2, ready_gemm12=ready_gemm12, cooperative=cooperative,
                     max_microbatches=3)


def test_deferred_weight_gradients_slot_limit():
    # more launches than slots before the experts are applied is refused, and
    # the handle stays usable: the next update from a zeroing launch matches
    cfg = synth.small_config("deferred_limit", 512, 128, 256, 8, 2, "bf16", microbatches=3)
    inp = synth.make_inputs(cfg, 24)
    run = GpuRun(cfg, inp, wg_per_cu=2, max_microbatches=2)
    try:
        x, t = run.microbatch(0)
        L = run.layer
        L.run(x, t, tokens_in_update=3 * cfg.tokens, step=1, zero_grad=True, apply=False)
        L.run(x, t, tokens_in_update=3 * cfg.tokens, step=1, zero_grad=False, apply=False)
        with pytest.raises(B.MoeStepError) as ei:
            L.run(x, t, tokens_in_update=3 * cfg.tokens, step=1, zero_grad=False, apply=False)
        assert ei.value.status == B.MOE_ERR_STATE
        torch.cuda.synchronize()
        L.status()
    finally:
        run.close()
    cfg2 = synth.small_config("deferred_limit", 512, 128, 256, 8, 2, "bf16", microbatches=2)
    _run_and_compare(cfg2, synth.make_inputs(cfg2, 24), BF16_TOL, steps=1, wg_per_cu=2, max_microbatches=2)


@pytest.mark.timeout(1200)
def test_zipf_16x8x1024_accumulated_deferred_weight_gradients():
    cfg = synth.CONFIGS["zipf_16x8x1024"]
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL, steps=1, max_microbatches=cfg.microbatches)


@pytest.mark.timeout(1200)
def test_zipf_16x8x1024_accumulated_full_size():
    cfg = synth.CONFIGS["zipf_16x8x1024"]
    inp = synth.make_inputs(cfg, 0)
    _run_and_compare(cfg, inp, BF16_TOL, steps=1)


@pytest.mark.parametrize("dtype,T,d,f,E,k,wg_per_cu", [("f32", 1000, 128, 64, 3, 2, 1),
                                                       ("f32", 777, 256, 136, 20, 3, 1),
                                                       ("bf16", 1000, 128, 64, 16, 2, 1),
                                                       ("bf16", 999, 384, 128, 20, 4, 2),
                                                       ("bf16", 513, 256, 128, 64, 8, 1),
                                                       ("bf16", 40000, 128, 64, 12, 2, 2),
                                                       ("bf16", 18000, 128, 64, 16, 2, 1)])
def test_router_on_matrix_cores(dtype, T, d, f, E, k, wg_per_cu):
    # d a multiple of 128: router logits by 16x16 fp32 matrix products, the
    # contraction split over the 4 waves; expert counts that leave padded
    # columns (3, 20, 12), four expert tiles (E = 64), and token ranges of
    # more than 64 per workgroup (several blocks of token tiles)
    cfg = synth.small_config(f"router_mfma_{dtype}", T, d, f, E, k, dtype)
    _run_and_compare(cfg, synth.make_inputs(cfg, 12), BF16_TOL if dtype == "bf16" else F32_TOL, steps=1,
                     wg_per_cu=wg_per_cu)


@pytest.mark.parametrize("wg_per_cu,T,d", [(1, 16 * 256 + 352, 96), (2, 16 * 512 + 704, 96), (1, 3000, 256),
                                           (2, 3000, 256)])
def test_routing_exact_ties_bf16_several_tokens_per_lane(wg_per_cu, T, d):
    # bf16 activations on the router path that gives each lane several tokens
    # (at least 16 tokens per workgroup pass; d = 256 takes the matrix-core
    # path): duplicated router columns give bitwise-equal logits, so the lower
    # expert index must win every tie
    cfg = synth.small_config(f"ties_bf16_occ{wg_per_cu}_d{d}", T, d, 64, 12, 2, "bf16")
    inp = synth.make_inputs(cfg, 16)
    pairs = ((1, 3), (0, 5), (7, 11))
    for lo, hi in pairs:
        inp.w_router[:, hi] = inp.w_router[:, lo]
    run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu)
    try:
        out = run.update(1)
        z, idx = out["logits"][0], out["idx"][0]
        decided = 0
        for lo, hi in pairs:
            assert np.array_equal(z[:, lo], z[:, hi]), "duplicated router columns must give equal logits"
            sel_lo = (idx == lo).any(axis=1)
            sel_hi = (idx == hi).any(axis=1)
            assert not np.any(sel_hi & ~sel_lo), "a tied higher index was chosen over the lower one"
            decided += int(np.sum(sel_lo & ~sel_hi))
        say(f"  tokens whose choice was decided by an exact tie: {decided}")
        assert decided > 0
        _check_routing(cfg, inp, out, inp.w_router.astype(np.float64))
        params = inp.flat_params().astype(np.float64)
        ref = oracle_update(cfg, inp, params, np.zeros_like(params), np.zeros_like(params), 1, out["idx"])
        errs, bad = compare_update(cfg, out, ref, **BF16_TOL,
                                   prev=(params, np.zeros_like(params), np.zeros_like(params), 1, cfg.clip_norm))
        assert not bad, f"{bad}: {errs}"
    finally:
        run.close()


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_forced_shadow_refresh_is_bit_identical(wg_per_cu):
    # AdamW writes the bf16 weight copy with the same round-to-nearest-even
    # conversion that MOE_RUN_REFRESH_SHADOW uses, so forcing a refresh before
    # the second update must change no bit of any output
    cfg = synth.small_config("shadow_bf16", 1000, 256, 384, 16, 2, "bf16")
    inp = synth.make_inputs(cfg, 17)
    outs = []
    for force in (False, True):
        run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu)
        try:
            run.update(1)
            L = run.layer
            dx = torch.empty(cfg.tokens, cfg.d_model, dtype=torch.float32, device=run.dev)
            L.run(run.x, run.t, step=2, dx=dx, refresh_shadow=force)
            L.status()
            torch.cuda.synchronize()
            outs.append({"grads": L.grads.cpu().numpy(), "params": L.params.cpu().numpy(),
                         "exp_avg": L.exp_avg.cpu().numpy(), "exp_avg_sq": L.exp_avg_sq.cpu().numpy(),
                         "dx": dx.cpu().numpy(), "stats": L.stats.cpu().numpy()})
        finally:
            run.close()
    for key in outs[0]:
        assert np.array_equal(outs[0][key], outs[1][key]), key


@pytest.mark.parametrize("dtype,wg_per_cu", [("f32", 1), ("bf16", 1), ("bf16", 2)])
def test_barrier_timeout_reported_and_handle_recovers(dtype, wg_per_cu):
    # The failure-path test flag makes one workgroup give up before the first
    # grid barrier (a wait on a word nothing sets, bounded at about 10 us), so
    # every other workgroup's barrier wait gives up as well and all exit.  A
    # launch enqueued behind it, before moe_step_status, must write nothing; the
    # status call reports the timeout bit and resets the barrier state; the
    # next update on the same handle matches the oracle.
    cfg = synth.small_config(f"timeout_{dtype}", 1000, 256, 384, 16, 2, dtype)
    inp = synth.make_inputs(cfg, 18)
    run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu)
    try:
        L = run.layer
        say(f"  [gpu] test-timeout launch, {dtype} wg_per_cu={wg_per_cu}")
        L.run(run.x, run.t, step=1, test_timeout=True)
        sentinel = 12345.0
        L.grads.fill_(sentinel)
        torch.cuda.synchronize()
        p_before = L.params.cpu().numpy()
        dx = torch.full((cfg.tokens, cfg.d_model), sentinel, dtype=torch.float32, device=run.dev)
        L.run(run.x, run.t, step=1, dx=dx)   # behind the failed launch: must write nothing
        with pytest.raises(B.MoeStepError) as ei:
            L.status()
        assert ei.value.status == B.MOE_ERR_DEVICE
        assert "grid-barrier timeout" in str(ei.value)
        torch.cuda.synchronize()
        assert np.all(L.grads.cpu().numpy() == sentinel)
        assert np.all(dx.cpu().numpy() == sentinel)
        assert np.array_equal(L.params.cpu().numpy(), p_before)
        L.status()   # the state was reset: no error now
        L.load_params(torch.from_numpy(inp.flat_params()))
        out = run.update(1)
        params = inp.flat_params().astype(np.float64)
        z = np.zeros_like(params)
        ref = oracle_update(cfg, inp, params, z, z, 1, out["idx"])
        errs, bad = compare_update(cfg, out, ref, **(BF16_TOL if dtype == "bf16" else F32_TOL),
                                   prev=(params, z, z, 1, cfg.clip_norm))
        assert not bad, f"update after the reported timeout: {bad}: {errs}"
    finally:
        run.close()


# ----------------------------------------------------------------------------
# Memory rule: recomputation (only H of the first expert product is stored)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,T,d,f,E,k,wg_per_cu,mb,skew", [
    ("f32", 333, 72, 136, 5, 2, 1, 1, False),
    ("bf16", 333, 72, 136, 5, 2, 1, 1, False),
    ("bf16", 1000, 256, 384, 16, 2, 1, 1, False),
    ("bf16", 1000, 256, 384, 16, 2, 2, 1, False),
    ("bf16", 300, 128, 64, 64, 8, 2, 1, False),
    # split weight-gradient contractions (partial dW2 tiles also recompute gelu(H))
    ("bf16", 1000, 256, 384, 16, 2, 1, 2, True),
    ("f32", 300, 72, 136, 5, 2, 1, 3, True),
])
def test_recompute_rule(dtype, T, d, f, E, k, wg_per_cu, mb, skew):
    # GEMM 1 keeps H only; GEMM 2 and dW2 apply GELU to their A fragments, the
    # dH epilogue forms gelu'(H): the same update within the same gates
    cfg = synth.small_config(f"recompute_{dtype}", T, d, f, E, k, dtype, microbatches=mb)
    inp = synth.make_inputs(cfg, 19)
    if skew:
        bias = np.zeros(E, np.float32)
        bias[0], bias[1] = 4.0, 2.0
        inp.router_bias = bias
    _run_and_compare(cfg, inp, BF16_TOL if dtype == "bf16" else F32_TOL, steps=2, wg_per_cu=wg_per_cu,
                     memory_rules=B.MOE_MEM_RECOMPUTE)


def test_recompute_rule_arena_and_2x1024():
    # the 2x1024 workload under the rule, and the arena it saves: one
    # [tokens * top_k, d_ff] bf16 tensor
    cfg = synth.CONFIGS["bf16_2x1024"]
    sizes = []
    for rules in (0, B.MOE_MEM_RECOMPUTE):
        from moe_step_megakernel_amd.layer import MoeLayerStep
        L = MoeLayerStep(cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, cfg.tokens, "bf16", memory_rules=rules)
        sizes.append(L.arena_bytes())
        L.close()
    saved = sizes[0] - sizes[1]
    say(f"  arena {sizes[0]} -> {sizes[1]} bytes")
    assert saved >= cfg.tokens * cfg.top_k * cfg.d_ff * 2 - 256   # less one 256-byte alignment unit
    _run_and_compare(cfg, synth.make_inputs(cfg, 0), BF16_TOL, steps=1, memory_rules=B.MOE_MEM_RECOMPUTE)
