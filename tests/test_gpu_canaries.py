"""Guard zones around every caller-owned buffer and inside the arena, on an MI355X.  Each buffer that
an update reads or writes through the C ABI (weights, gradients, moments,
stats, dx, the debug outputs, the phase trace; x, target and the router bias)
is the middle of a larger allocation whose head and tail hold a fill pattern.
After whole updates on ragged shapes, top-8 routing, skewed routing with
split and deferred weight-gradient contractions, both occupancies and fp32,
every guard word must still hold the pattern and the inputs must be unchanged:
the kernels write only inside the outputs they are given.  The results
themselves are checked against the oracle elsewhere; here only that the
update ran (finite loss, moved weights, written debug outputs).  The pattern
is a quiet NaN, so a read past the end of an input that reached a result would
also show, as a non-finite dx, loss or weight."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import GpuRun, say
from moe_step_megakernel_amd import binding as B

pytestmark = pytest.mark.gpu

GUARD = 4096                 # guard words on each side of a buffer
PATTERN = 0x7FC0DEAD         # a quiet-NaN bit pattern (int32 view)


class Guarded:
    """A contiguous view of the given shape in the middle of an allocation with
    GUARD words of fill pattern before and after it (16 KiB each, so the view
    keeps the allocation's alignment)."""

    def __init__(self, name, shape, dtype, dev):
        self.name = name
        self.nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.big = torch.empty((self.nbytes + 3) // 4 + 2 * GUARD, dtype=torch.int32, device=dev)
        self.big.fill_(PATTERN)
        self.view = self.big.view(torch.uint8)[4 * GUARD:4 * GUARD + self.nbytes].view(dtype).view(shape)

    def check(self):
        """Every byte before the view and from its last byte on (the padding of
        its last word included) still holds the pattern."""
        raw = self.big.view(torch.uint8).cpu().numpy()
        want = np.resize(np.frombuffer(np.array([PATTERN], "<i4").tobytes(), np.uint8), raw.size)
        for side, lo, hi in (("head", 0, 4 * GUARD), ("tail", 4 * GUARD + self.nbytes, raw.size)):
            bad = np.flatnonzero(raw[lo:hi] != want[lo:hi])
            assert bad.size == 0, f"{self.name}: {bad.size} guard bytes of the {side} overwritten (first at {bad[0]})"


def _guard_layer(run, dev, keep):
    """Moves the layer's own state tensors into guarded allocations."""
    L = run.layer
    for name in ("params", "grads", "exp_avg", "exp_avg_sq", "stats"):
        old = getattr(L, name)
        g = Guarded(name, tuple(old.shape), old.dtype, dev)
        g.view.copy_(old)
        setattr(L, name, g.view)
        keep.append(g)


def _run_guarded(cfg, inp, *, wg_per_cu=0, max_microbatches=0, trace=False):
    say(f"[gpu] canaries {cfg.name} T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} "
        f"E={cfg.n_experts} k={cfg.top_k} {cfg.dtype} wg_per_cu={wg_per_cu} deferred={max_microbatches}")
    run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu, max_microbatches=max_microbatches)
    dev = run.dev
    L = run.layer
    T, E, k, d = cfg.tokens, cfg.n_experts, cfg.top_k, cfg.d_model
    act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32   # inputs compared bit for bit
    guards = []
    try:
        _guard_layer(run, dev, guards)
        p0 = L.params.clone()
        bias = None
        if run.bias is not None:
            gb = Guarded("router_bias", (E,), torch.float32, dev)
            gb.view.copy_(run.bias)
            bias, bias0 = gb.view, run.bias.clone()
            guards.append(gb)
        for step in (1, 2):
            for mb in range(cfg.microbatches):
                x0, t0 = run.microbatch(mb)
                gx, gt = Guarded("x", (T, d), act, dev), Guarded("target", (T, d), act, dev)
                gx.view.copy_(x0)
                gt.view.copy_(t0)
                gdx = Guarded("dx", (T, d), torch.float32, dev)
                dbg = {"router_logits": Guarded("router_logits", (T, E), torch.float32, dev),
                       "topk_idx": Guarded("topk_idx", (T, k), torch.int32, dev),
                       "topk_gate": Guarded("topk_gate", (T, k), torch.float32, dev),
                       "expert_counts": Guarded("expert_counts", (E,), torch.int32, dev),
                       "route_perm": Guarded("route_perm", (T * k,), torch.int32, dev)}
                gtr = Guarded("trace", (L.trace_words(),), torch.int64, dev) if trace else None
                L.run(gx.view, gt.view, tokens_in_update=cfg.tokens_in_update, step=step, zero_grad=(mb == 0),
                      apply=(mb == cfg.microbatches - 1), dx=gdx.view, router_bias=bias,
                      debug={n: g.view for n, g in dbg.items()}, trace=None if gtr is None else gtr.view)
                L.status()
                torch.cuda.synchronize()
                for g in [gx, gt, gdx, *dbg.values()] + ([gtr] if gtr is not None else []):
                    g.check()
                # the inputs are read only
                assert torch.equal(gx.view.view(bits), x0.contiguous().view(bits))
                assert torch.equal(gt.view.view(bits), t0.contiguous().view(bits))
                # the update ran: every token has k distinct experts, the counts add up
                idx = dbg["topk_idx"].view.cpu().numpy()
                assert idx.min() >= 0 and idx.max() < E
                assert all(len(set(r)) == k for r in idx[: min(T, 64)])
                assert int(dbg["expert_counts"].view.sum().item()) == T * k
                assert torch.isfinite(gdx.view).all()
            for g in guards:
                g.check()
            if bias is not None:
                assert torch.equal(bias, bias0)
            loss = float(L.stats[0].item())
            assert np.isfinite(loss) and loss > 0.0, loss
        assert not torch.equal(L.params, p0), "the weights did not move"
        assert torch.isfinite(L.params).all() and torch.isfinite(L.exp_avg_sq).all()
        say(f"  guards intact, loss {loss:.5f}")
    finally:
        run.close()


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_guards_bf16_ragged_with_trace(wg_per_cu):
    cfg = synth.small_config(f"canary_bf16_occ{wg_per_cu}", 1000, 256, 384, 16, 2, "bf16")
    _run_guarded(cfg, synth.make_inputs(cfg, 31), wg_per_cu=wg_per_cu, trace=True)


def test_guards_top8():
    cfg = synth.small_config("canary_top8", 300, 128, 64, 64, 8, "bf16")
    _run_guarded(cfg, synth.make_inputs(cfg, 32))


def test_guards_fp32_ragged():
    cfg = synth.small_config("canary_f32", 201, 72, 136, 6, 2, "f32")
    _run_guarded(cfg, synth.make_inputs(cfg, 33))


@pytest.mark.parametrize("deferred", [0, 3])
def test_guards_skewed_accumulated(deferred):
    # skewed routing splits the weight-gradient contractions; with deferral the
    # applying launch contracts over the three microbatch slots
    cfg = synth.small_config("canary_skewed", 768, 256, 384, 16, 2, "bf16", microbatches=3)
    inp = synth.make_inputs(cfg, 34)
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[0], bias[1] = 4.0, 2.0
    inp.router_bias = bias
    _run_guarded(cfg, inp, wg_per_cu=2, max_microbatches=deferred)


# ---------------------------------------------------------------------------
# Guard zones inside the library's arena (memory_rules MOE_MEM_GUARDS): every
# sub-buffer is followed by a zone of at least 1 MiB that must stay zero.  The
# same updates run on a plain handle and on a guarded one; the guarded layout
# moves the sub-buffers apart and must change no result bit.
# ---------------------------------------------------------------------------

def _update_outputs(run, steps):
    outs = []
    for step in steps:
        o = run.update(step)
        outs.append({key: (np.concatenate([np.asarray(a).ravel() for a in v]) if isinstance(v, list) else np.atleast_1d(v))
                     for key, v in o.items()})
    return outs


def _arena_guards(cfg, inp, *, wg_per_cu=0, max_microbatches=0, memory_rules=0, ready_gemm12=False):
    say(f"[gpu] arena guards {cfg.name} T={cfg.tokens}x{cfg.microbatches} d={cfg.d_model} f={cfg.d_ff} "
        f"E={cfg.n_experts} k={cfg.top_k} {cfg.dtype} wg_per_cu={wg_per_cu} deferred={max_microbatches} "
        f"rules={memory_rules} ready12={ready_gemm12}")
    results, sizes = [], []
    for rules in (memory_rules, memory_rules | B.MOE_MEM_GUARDS):
        run = GpuRun(cfg, inp, wg_per_cu=wg_per_cu, max_microbatches=max_microbatches, memory_rules=rules,
                     ready_gemm12=ready_gemm12)
        try:
            results.append(_update_outputs(run, (1, 2)))
            sizes.append(run.layer.arena_bytes())
            if rules & B.MOE_MEM_GUARDS:
                run.layer.check_guards()
        finally:
            run.close()
    assert sizes[1] > sizes[0] + (1 << 20) * 20, sizes
    for step, (a, b) in enumerate(zip(*results), start=1):
        for key in a:
            assert np.array_equal(np.asarray(a[key]).view(np.uint8), np.asarray(b[key]).view(np.uint8)), \
                f"update {step}: {key} differs between the plain and the guarded arena layout"
    say(f"  guard zones intact; results bitwise equal to the plain layout (arena {sizes[0]} -> {sizes[1]} bytes)")


@pytest.mark.parametrize("wg_per_cu", [1, 2])
def test_arena_guards_bf16_ragged(wg_per_cu):
    cfg = synth.small_config(f"arena_bf16_occ{wg_per_cu}", 1000, 256, 384, 16, 2, "bf16")
    _arena_guards(cfg, synth.make_inputs(cfg, 41), wg_per_cu=wg_per_cu)


def test_arena_guards_top8_readiness_counters():
    cfg = synth.small_config("arena_top8", 300, 128, 64, 64, 8, "bf16")
    _arena_guards(cfg, synth.make_inputs(cfg, 42), ready_gemm12=True)


def test_arena_guards_fp32_ragged():
    cfg = synth.small_config("arena_f32", 201, 72, 136, 6, 2, "f32")
    _arena_guards(cfg, synth.make_inputs(cfg, 43))


def test_arena_guards_recompute_rule():
    cfg = synth.small_config("arena_recompute", 1000, 256, 384, 16, 2, "bf16")
    _arena_guards(cfg, synth.make_inputs(cfg, 44), memory_rules=B.MOE_MEM_RECOMPUTE)


@pytest.mark.parametrize("deferred", [0, 3])
def test_arena_guards_skewed_accumulated(deferred):
    cfg = synth.small_config("arena_skewed", 768, 256, 384, 16, 2, "bf16", microbatches=3)
    inp = synth.make_inputs(cfg, 45)
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[0], bias[1] = 4.0, 2.0
    inp.router_bias = bias
    _arena_guards(cfg, inp, wg_per_cu=2, max_microbatches=deferred)


def test_arena_guards_2x1024_shape():
    cfg = synth.CONFIGS["bf16_2x1024"]
    _arena_guards(cfg, synth.make_inputs(cfg, 0))
