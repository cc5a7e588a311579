"""The allocation-free entry point moe_step_run_static (arena in a static
device array, no handle) against moe_step_run on a handle with the same
configuration: two updates in a row, the second with fewer tokens, must give
bit-identical outputs (same kernel, same grid, deterministic order of every
sum), and the static call reports a clean device status in stats[3].  A
configuration whose arena does not fit the static array is refused on the
host."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_tokens, say
from moe_step_megakernel_amd import binding as B
from moe_step_megakernel_amd.layer import MoeLayerStep

pytestmark = pytest.mark.gpu


def _inputs(cfg, seed, dev):
    inp = synth.make_inputs(cfg, seed)
    return inp, device_tokens(inp.x, inp.x_bits, cfg.dtype, dev), device_tokens(inp.t, inp.t_bits, cfg.dtype, dev)


@pytest.mark.parametrize("dtype,wg_per_cu", [("bf16", 1), ("bf16", 2), ("f32", 1)])
def test_static_entry_matches_handle_entry(dtype, wg_per_cu):
    dev = torch.device("cuda", 0)
    d, f, E, k, tmax = 256, 384, 16, 2, 1000
    cfg0 = synth.small_config(f"static_{dtype}", tmax, d, f, E, k, dtype)
    inp0, x0, t0 = _inputs(cfg0, 31, dev)
    cfg1 = synth.small_config(f"static_{dtype}_small", 333, d, f, E, k, dtype)
    _, x1, t1 = _inputs(cfg1, 32, dev)
    calls = ((x0, t0, 1), (x1, t1, 2))
    say(f"[gpu] static entry {dtype} wg_per_cu={wg_per_cu}: {tmax} then 333 tokens")

    # the existing entry point: a handle with its own arena
    layer = MoeLayerStep(d, f, E, k, tmax, dtype, wg_per_cu=wg_per_cu)
    ref = []
    try:
        layer.load_params(torch.from_numpy(inp0.flat_params()))
        for x, t, step in calls:
            dx = torch.empty(x.shape[0], d, dtype=torch.float32, device=dev)
            layer.run(x, t, step=step, dx=dx)
            layer.status()
            torch.cuda.synchronize()
            ref.append({"grads": layer.grads.cpu().numpy(), "params": layer.params.cpu().numpy(),
                        "exp_avg": layer.exp_avg.cpu().numpy(), "exp_avg_sq": layer.exp_avg_sq.cpu().numpy(),
                        "dx": dx.cpu().numpy(), "stats": layer.stats[:3].cpu().numpy()})
        grid = layer.grid
    finally:
        layer.close()

    # the allocation-free entry point: caller tensors only
    cfg = B.make_config(d, f, E, k, tmax, dtype, wg_per_cu=wg_per_cu)
    P = B.moe_step_param_count(cfg)
    params = torch.from_numpy(inp0.flat_params()).to(dev)
    grads, m, v = (torch.zeros(P, dtype=torch.float32, device=dev) for _ in range(3))
    stats = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i, (x, t, step) in enumerate(calls):
        dx = torch.empty(x.shape[0], d, dtype=torch.float32, device=dev)
        io = B.make_io(x=x, target=t, params=params, grads=grads, exp_avg=m, exp_avg_sq=v, dx=dx, stats=stats)
        B.moe_step_run_static(cfg, io, x.shape[0], x.shape[0], step, B.MOE_RUN_ZERO_GRAD | B.MOE_RUN_APPLY,
                              stream.cuda_stream)
        torch.cuda.synchronize()
        st = stats.cpu().numpy()
        assert st[3] == 0.0, f"device status {st[3]}"
        got = {"grads": grads.cpu().numpy(), "params": params.cpu().numpy(), "exp_avg": m.cpu().numpy(),
               "exp_avg_sq": v.cpu().numpy(), "dx": dx.cpu().numpy(), "stats": st[:3]}
        for key in got:
            assert np.array_equal(got[key], ref[i][key]), f"call {i + 1}: {key} differs"
        say(f"  call {i + 1} ({x.shape[0]} tokens, grid {grid}): bit-identical to the handle entry point; "
            f"loss {st[0]:.6g}")


def test_static_entry_refuses_what_does_not_fit():
    dev = torch.device("cuda", 0)
    cfg = B.make_config(768, 1536, 16, 2, 2048, "bf16")   # arena of about 214 MB
    P = B.moe_step_param_count(cfg)
    z = torch.zeros(P, dtype=torch.float32, device=dev)
    stats = torch.zeros(4, dtype=torch.float32, device=dev)
    x = torch.zeros(2048, 768, dtype=torch.bfloat16, device=dev)
    io = B.make_io(x=x, target=x, params=z, grads=z, exp_avg=z, exp_avg_sq=z, stats=stats)
    with pytest.raises(B.MoeStepError) as ei:
        B.moe_step_run_static(cfg, io, 2048, 2048, 1, B.MOE_RUN_ZERO_GRAD | B.MOE_RUN_APPLY)
    assert ei.value.status == B.MOE_ERR_SHAPE
    assert "static scratch holds" in str(ei.value)
    io_nostats = B.make_io(x=x, target=x, params=z, grads=z, exp_avg=z, exp_avg_sq=z)
    with pytest.raises(B.MoeStepError) as ei:
        B.moe_step_run_static(B.make_config(64, 128, 4, 2, 256, "bf16"), io_nostats, 256, 256, 1, 0)
    assert ei.value.status == B.MOE_ERR_ARG
