"""The GPU parity gates themselves, on the CPU: identical outputs pass, and a
mistake planted in a copy of the oracle's own outputs is caught by the local
gates even where the whole-tensor relative L2 stays under its bound (a wrong
128 x 128 gradient tile among many, a wrong 128-token dx block, a wrong expert
slice of a moment, a wrong optimizer step in one expert)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import compare_update, rel_l2

BF16_TOL = dict(grad_tol=0.08, weight_tol=1e-2, loss_tol=1e-2)


@pytest.fixture(scope="module")
def case():
    # 8 experts of a 256 x 384 layer: dW1 has 2 x 3 tiles per expert, 48 in all
    cfg = synth.small_config("gates", 1024, 256, 384, 8, 2, "f32")
    inp = synth.make_inputs(cfg, 2)
    p = inp.flat_params().astype(np.float64)
    z = np.zeros_like(p)
    ref = oracle.step([inp.x], [inp.t], p, z, z, 1, d=cfg.d_model, f=cfg.d_ff, E=cfg.n_experts,
                      top_k=cfg.top_k)
    return cfg, ref, (p, z, z, 1, cfg.clip_norm)


def _copy(ref):
    out = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    out["dx"] = [np.array(ref["dx"], copy=True)]
    return out


def test_identical_outputs_pass(case):
    cfg, ref, prev = case
    _, bad = compare_update(cfg, _copy(ref), ref, **BF16_TOL, prev=prev)
    assert bad == []


def test_one_wrong_gradient_tile_is_caught(case):
    cfg, ref, prev = case
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    gpu = _copy(ref)
    w1 = gpu["grads"][d * E:d * E + E * d * f].reshape(E, d, f)
    w1[5, 128:256, 256:384] *= 1.3             # one tile of expert 5 is 30% off
    whole = rel_l2(gpu["grads"][d * E:d * E + E * d * f], ref["grads"][d * E:d * E + E * d * f])
    assert whole < 0.08                         # the whole-tensor gate alone would pass it
    _, bad = compare_update(cfg, gpu, ref, **BF16_TOL)
    assert any(b.startswith("dW1 expert 5 tile [128:256,256:384]") for b in bad), bad


def test_one_wrong_dx_block_is_caught(case):
    cfg, ref, prev = case
    gpu = _copy(ref)
    gpu["dx"][0][384:512] *= 1.2                # a 20% error on one 128-token block
    assert rel_l2(gpu["dx"][0], ref["dx"]) < 0.08
    _, bad = compare_update(cfg, gpu, ref, **BF16_TOL)
    assert "dx tokens[384:512] (0.2)" in bad, bad


def test_one_wrong_moment_slice_is_caught(case):
    cfg, ref, prev = case
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    gpu = _copy(ref)
    m = gpu["exp_avg"]
    m[d * E + 3 * d * f:d * E + 4 * d * f] *= 1.15   # expert 3 of the W1 first moment
    assert rel_l2(m, ref["exp_avg"]) < 0.08
    _, bad = compare_update(cfg, gpu, ref, **BF16_TOL, prev=prev)
    assert any(b.startswith("exp_avg.W1 expert 3") for b in bad), bad
    assert any(b.startswith("adamw_own.exp_avg.W1 expert 3") for b in bad), bad


def test_one_wrong_optimizer_step_is_caught(case):
    cfg, ref, prev = case
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    gpu = _copy(ref)
    p0 = prev[0]
    sl = slice(d * E + E * d * f + 6 * f * d, d * E + E * d * f + 7 * f * d)   # expert 6 of W2
    gpu["params"][sl] = p0[sl] + 0.5 * (ref["params"][sl] - p0[sl])            # half the step
    assert rel_l2(gpu["params"], ref["params"]) < 1e-2
    _, bad = compare_update(cfg, gpu, ref, **BF16_TOL, prev=prev)
    assert any(b.startswith("adamw_own.params.W2 expert 6") for b in bad), bad
