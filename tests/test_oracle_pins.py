"""Pins of the FP64 oracle to things other than itself (CPU only).

Each test states what fixes the expected value: a number printed on the Latch
pages, a closed form, a library routine on a special case, brute force on tiny
inputs, or an invariant of the mathematics.  A plausible mistake in the oracle
(a dropped term, a wrong sign or index, a transposed operand) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# Worked example: "How a training megakernel works", "One training update"
# ----------------------------------------------------------------------------
def _worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        doc = json.load(fh)
    i = doc["inputs"]
    # E = 1 expert, top-1 (the gate is a softmax over one logit, so it is 1),
    # d = f = 1, identity activation, plain SGD, no clipping, one token.
    params = np.array([0.0, i["w1"], i["w2"]])    # W_r | W1 | W2
    out = oracle.step(np.array([[i["x"]]]), np.array([[i["t"]]]), params, np.zeros(3), np.zeros(3), 1,
                      d=1, f=1, E=1, top_k=1, lr=i["eta"], clip_norm=0.0, act="identity", opt="sgd",
                      with_loss_after=True)
    return doc, out


def test_worked_example_forward_loss_gradients():
    doc, out = _worked_example()
    p = doc["printed"]
    assert out["loss"] == pytest.approx(p["loss"], abs=1e-15)
    assert out["grads"][1] == pytest.approx(p["dL_dw1"], abs=1e-15)
    assert out["grads"][2] == pytest.approx(p["dL_dw2"], abs=1e-15)
    assert out["grads"][0] == 0.0                      # router gradient vanishes with one expert
    assert float(out["dx"][0, 0]) == pytest.approx(doc["derived_not_printed"]["dL_dx"], abs=1e-15)


def test_worked_example_update_and_loss_after():
    doc, out = _worked_example()
    p = doc["printed"]
    assert out["params"][1] == pytest.approx(p["w1_after"], abs=1e-15)
    assert out["params"][2] == pytest.approx(p["w2_after"], abs=1e-15)
    assert out["loss_after"] == pytest.approx(doc["exact"]["loss_after"], rel=1e-12)
    assert round(out["loss_after"], 5) == p["loss_after_printed_rounded"]


def test_worked_example_intermediates():
    doc, _ = _worked_example()
    i, p = doc["inputs"], doc["printed"]
    fw = oracle.layer_forward(np.array([[i["x"]]]), np.array([[i["t"]]]), np.zeros((1, 1)),
                              np.array([[[i["w1"]]]]), np.array([[[i["w2"]]]]), 1, 1, act="identity")
    assert fw["H"][0, 0] == p["h"]
    assert fw["y"][0, 0] == p["y"]
    fw2 = oracle.layer_forward(np.array([[i["x"]]]), np.array([[i["t"]]]), np.zeros((1, 1)),
                               np.array([[[p["w1_after"]]]]), np.array([[[p["w2_after"]]]]), 1, 1,
                               act="identity")
    assert fw2["H"][0, 0] == pytest.approx(p["h_after"], abs=1e-15)
    assert fw2["y"][0, 0] == pytest.approx(p["y_after"], abs=1e-15)


# ----------------------------------------------------------------------------
# GELU (tanh form) against PyTorch's library routine in float64
# ----------------------------------------------------------------------------
def test_gelu_matches_library_and_closed_values():
    h = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.tensor(h, dtype=torch.float64), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(h), ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(30.0) == pytest.approx(30.0, rel=1e-15)
    assert abs(oracle.gelu_tanh(-30.0)) < 1e-300 or oracle.gelu_tanh(-30.0) == pytest.approx(0.0, abs=1e-12)


def test_gelu_grad_matches_library_autograd():
    h = torch.tensor(np.linspace(-6, 6, 1201), dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(h, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(h.detach().numpy()), h.grad.numpy(), rtol=1e-13, atol=1e-14)
    assert oracle.gelu_tanh_grad(0.0) == 0.5


# ----------------------------------------------------------------------------
# token_topk against the brute-force rank definition
# ----------------------------------------------------------------------------
def _brute_topk(z, k):
    T, E = z.shape
    out = np.empty((T, k), np.int64)
    for i in range(T):
        rank = {}
        for e in range(E):
            rank[e] = sum(1 for e2 in range(E) if z[i, e2] > z[i, e] or (z[i, e2] == z[i, e] and e2 < e))
        for e, r in rank.items():
            if r < k:
                out[i, r] = e
    return out


@pytest.mark.parametrize("E,k", [(4, 2), (16, 2), (8, 8), (64, 8), (5, 1), (3, 3)])
def test_token_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    z_int = rng.integers(-2, 3, size=(200, E)).astype(np.float64)   # many exact ties
    z_real = rng.standard_normal((200, E))
    for z in (z_int, z_real):
        np.testing.assert_array_equal(oracle.token_topk(z, k), _brute_topk(z, k))


def test_token_topk_signed_zero_ties_and_nan():
    z = np.array([[0.0, -0.0, -1.0, 0.0], [-0.0, 0.0, 0.0, -0.0]])
    np.testing.assert_array_equal(oracle.token_topk(z, 2), [[0, 1], [0, 1]])
    with pytest.raises(ValueError):
        oracle.token_topk(np.array([[0.0, np.nan]]), 1)


def test_gates_are_renormalised_full_softmax():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 16)) * 3
    sel = oracle.token_topk(z, 2)
    g = oracle.topk_gates(z, sel)
    full = np.exp(z - z.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    picked = np.take_along_axis(full, sel, axis=1)
    np.testing.assert_allclose(g, picked / picked.sum(axis=1, keepdims=True), rtol=1e-14)
    assert np.all(g[:, 0] >= g[:, 1])


# ----------------------------------------------------------------------------
# route_order against brute force, and its invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(37, 4, 2), (100, 16, 2), (20, 64, 8), (9, 3, 3), (1, 1, 1)])
def test_route_order_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    sel = oracle.token_topk(rng.standard_normal((T, E)), k)
    counts, offsets, perm, inv = oracle.route_order(sel, E)
    flat = sel.reshape(-1)
    N = T * k
    assert counts.sum() == N and offsets[0] == 0 and offsets[-1] == N
    for q in range(N):
        e = flat[q]
        pos = offsets[e] + sum(1 for q2 in range(q) if flat[q2] == e)
        assert inv[q] == pos and perm[pos] == q
    assert sorted(perm.tolist()) == list(range(N))
    np.testing.assert_array_equal(inv[perm], np.arange(N))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                  # stable: ascending flat id
        assert np.all(flat[seg] == e)


def test_route_order_empty_experts():
    sel = np.array([[2, 0], [2, 0], [0, 2]])
    counts, offsets, perm, inv = oracle.route_order(sel, 5)
    np.testing.assert_array_equal(counts, [3, 0, 3, 0, 0])
    np.testing.assert_array_equal(offsets, [0, 3, 3, 6, 6, 6])
    np.testing.assert_array_equal(perm, [1, 3, 4, 0, 2, 5])


# ----------------------------------------------------------------------------
# Whole layer: central finite differences
# ----------------------------------------------------------------------------
def _tiny(T, d, f, E, k, seed, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    t = rng.standard_normal((T, d))
    params = np.concatenate([rng.standard_normal(d * E) * 0.8, rng.standard_normal(2 * E * d * f) * 0.5])
    b = rng.standard_normal(E) * 0.3 if bias else None
    return x, t, params, b


def _margin_ok(x, params, d, f, E, k, b, h):
    w_r, _, _ = oracle.unpack_params(params, d, f, E)
    z = oracle.router_logits(x, w_r, b)
    zs = np.sort(z, axis=1)[:, ::-1]
    if k == E:
        return True
    return np.min(zs[:, k - 1] - zs[:, k]) > 1e-3


@pytest.mark.parametrize("T,d,f,E,k,act,bias", [
    (8, 4, 6, 3, 2, "gelu_tanh", False),
    (8, 4, 6, 3, 1, "gelu_tanh", True),
    (6, 3, 5, 1, 1, "gelu_tanh", False),
    (7, 4, 4, 3, 3, "gelu_tanh", False),
    (8, 4, 6, 4, 2, "identity", False),
])
def test_gradients_central_finite_differences(T, d, f, E, k, act, bias):
    seed = 0
    while True:
        x, t, params, b = _tiny(T, d, f, E, k, seed, bias)
        if _margin_ok(x, params, d, f, E, k, b, 1e-6):
            break
        seed += 1
    kw = dict(d=d, f=f, E=E, top_k=k, bias=b, act=act)
    out = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, clip_norm=0.0, **kw)
    base_sel = out["routing"]["sel"]
    h = 1e-6

    def loss_at(p, xx):
        fw_sel = oracle.token_topk(oracle.router_logits(xx, oracle.unpack_params(p, d, f, E)[0], b), k)
        assert np.array_equal(fw_sel, base_sel), "routing changed under the perturbation"
        return oracle.forward_loss(xx, t, p, **kw)

    fd = np.empty_like(params)
    for i in range(params.size):
        pp, pm = params.copy(), params.copy()
        pp[i] += h
        pm[i] -= h
        fd[i] = (loss_at(pp, x) - loss_at(pm, x)) / (2 * h)
    n_r, n_1 = d * E, E * d * f
    for name, sl in (("dW_r", slice(0, n_r)), ("dW1", slice(n_r, n_r + n_1)), ("dW2", slice(n_r + n_1, None))):
        a, r = out["grads"][sl], fd[sl]
        if np.linalg.norm(r) == 0:
            assert np.linalg.norm(a) < 1e-12, name
            continue
        assert np.linalg.norm(a - r) / np.linalg.norm(r) < 1e-6, name
    fdx = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fdx[idx] = (loss_at(params, xp) - loss_at(params, xm)) / (2 * h)
    assert np.linalg.norm(out["dx"] - fdx) / np.linalg.norm(fdx) < 1e-6


# ----------------------------------------------------------------------------
# Special case: one expert, top-1 is a dense two-layer MLP (library autograd)
# ----------------------------------------------------------------------------
def test_single_expert_is_dense_mlp():
    rng = np.random.default_rng(11)
    T, d, f = 13, 5, 7
    x, t = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w1, w2 = rng.standard_normal((d, f)), rng.standard_normal((f, d))
    params = np.concatenate([rng.standard_normal(d), w1.ravel(), w2.ravel()])
    out = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1,
                      d=d, f=f, E=1, top_k=1, clip_norm=0.0)
    tx = torch.tensor(x, requires_grad=True)
    tw1 = torch.tensor(w1, requires_grad=True)
    tw2 = torch.tensor(w2, requires_grad=True)
    y = torch.nn.functional.gelu(tx @ tw1, approximate="tanh") @ tw2
    loss = 0.5 * ((y - torch.tensor(t)) ** 2).sum() / T
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-13)
    np.testing.assert_allclose(out["grads"][d:d + d * f], tw1.grad.numpy().ravel(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(out["grads"][d + d * f:], tw2.grad.numpy().ravel(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(out["dx"], tx.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.all(out["grads"][:d] == 0.0)


# ----------------------------------------------------------------------------
# The routed combine against a dense formulation (every token through every
# expert, then a masked, renormalised softmax over all E logits), via PyTorch
# autograd in float64 -- a different computation of the same layer.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("E,k", [(4, 2), (6, 3), (5, 1)])
def test_routed_layer_equals_dense_masked_formulation(E, k):
    rng = np.random.default_rng(E * 7 + k)
    T, d, f = 17, 6, 5
    x, t = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, E))
    w1 = rng.standard_normal((E, d, f)) * 0.7
    w2 = rng.standard_normal((E, f, d)) * 0.7
    params = oracle.pack(w_r, w1, w2)
    out = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1,
                      d=d, f=f, E=E, top_k=k, clip_norm=0.0)
    fw = oracle.layer_forward(x, t, w_r, w1, w2, k, T)

    tx = torch.tensor(x, requires_grad=True)
    tr = torch.tensor(w_r, requires_grad=True)
    t1 = torch.tensor(w1, requires_grad=True)
    t2 = torch.tensor(w2, requires_grad=True)
    z = tx @ tr
    mask = torch.zeros(T, E, dtype=torch.float64)
    for i in range(T):                              # selection from the brute-force rank rule
        for e in _brute_topk(z.detach().numpy()[i:i + 1], k)[0]:
            mask[i, e] = 1.0
    soft = torch.softmax(z, dim=1) * mask
    G = soft / soft.sum(dim=1, keepdim=True)
    ys = []
    for e in range(E):                               # dense: every token through expert e
        ys.append(torch.nn.functional.gelu(tx @ t1[e], approximate="tanh") @ t2[e])
    y = sum(G[:, e:e + 1] * ys[e] for e in range(E))
    loss = 0.5 * ((y - torch.tensor(t)) ** 2).sum() / T
    loss.backward()
    np.testing.assert_allclose(fw["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    got = oracle.unpack_params(out["grads"], d, f, E)
    for a, ref in zip(got, (tr.grad, t1.grad, t2.grad)):
        np.testing.assert_allclose(a, ref.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-13)


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------
def test_identical_experts_give_dense_output_and_no_router_gradient():
    rng = np.random.default_rng(5)
    T, d, f, E, k = 20, 6, 8, 4, 2
    x, t = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w1e, w2e = rng.standard_normal((d, f)), rng.standard_normal((f, d))
    w_r = rng.standard_normal((d, E))
    w1 = np.repeat(w1e[None], E, axis=0)
    w2 = np.repeat(w2e[None], E, axis=0)
    params = oracle.pack(w_r, w1, w2)
    out = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, d=d, f=f, E=E,
                      top_k=k, clip_norm=0.0)
    fw = oracle.layer_forward(x, t, w_r, w1, w2, k, T)
    dense = oracle.gelu_tanh(x @ w1e) @ w2e
    np.testing.assert_allclose(fw["y"], dense, rtol=1e-12, atol=1e-13)
    gr, g1, g2 = oracle.unpack_params(out["grads"], d, f, E)
    assert np.abs(gr).max() < 1e-13 * max(1.0, np.abs(g1).max())
    dense_out = oracle.step(x, t, np.concatenate([np.zeros(d), w1e.ravel(), w2e.ravel()]), np.zeros(d + 2 * d * f),
                            np.zeros(d + 2 * d * f), 1, d=d, f=f, E=1, top_k=1, clip_norm=0.0)
    _, dg1, dg2 = oracle.unpack_params(dense_out["grads"], d, f, 1)
    np.testing.assert_allclose(g1.sum(axis=0), dg1[0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g2.sum(axis=0), dg2[0], rtol=1e-11, atol=1e-13)


def test_token_permutation_equivariance():
    x, t, params, _ = _tiny(24, 6, 7, 5, 2, 9)
    kw = dict(d=6, f=7, E=5, top_k=2, clip_norm=0.0)
    a = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, **kw)
    pi = np.random.default_rng(1).permutation(24)
    b = oracle.step(x[pi], t[pi], params, np.zeros_like(params), np.zeros_like(params), 1, **kw)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-13)
    np.testing.assert_allclose(a["grads"], b["grads"], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(a["dx"][pi], b["dx"], rtol=1e-12, atol=1e-15)


def test_zero_residual_gives_zero_loss_and_gradients():
    x, _, params, _ = _tiny(10, 4, 6, 3, 2, 2)
    w_r, w1, w2 = oracle.unpack_params(params, 4, 6, 3)
    y = oracle.layer_forward(x, np.zeros_like(x), w_r, w1, w2, 2, 10)["y"]
    out = oracle.step(x, y, params, np.zeros_like(params), np.zeros_like(params), 1, d=4, f=6, E=3, top_k=2,
                      clip_norm=1.0)
    assert out["loss"] == 0.0
    assert np.all(out["grads"] == 0.0) and np.all(out["dx"] == 0.0)
    # with zero gradient AdamW only decays: w <- w (1 - lr wd)
    np.testing.assert_allclose(out["params"], params * (1 - 1e-3 * 0.01), rtol=1e-15)


def test_microbatch_accumulation_equals_one_batch():
    x, t, params, _ = _tiny(64, 6, 8, 4, 2, 4)
    kw = dict(d=6, f=8, E=4, top_k=2, clip_norm=0.5)
    one = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 3, **kw)
    acc = oracle.step([x[i * 16:(i + 1) * 16] for i in range(4)], [t[i * 16:(i + 1) * 16] for i in range(4)],
                      params, np.zeros_like(params), np.zeros_like(params), 3, **kw)
    assert acc["loss"] == pytest.approx(one["loss"], rel=1e-13)
    np.testing.assert_allclose(acc["grads"], one["grads"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(np.concatenate(acc["dx"]), one["dx"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(acc["params"], one["params"], rtol=1e-13)


# ----------------------------------------------------------------------------
# Clipping and AdamW closed forms
# ----------------------------------------------------------------------------
def test_clip_closed_form():
    g = np.random.default_rng(0).standard_normal(1000)
    n = oracle.global_norm([g])
    assert n == pytest.approx(math.sqrt(float(np.dot(g, g))), rel=1e-14)
    c = oracle.clip_coefficient(n, 1.0)
    assert np.linalg.norm(c * g) == pytest.approx(1.0 * n / (n + 1e-6), rel=1e-13)
    assert oracle.clip_coefficient(0.5, 1.0) == 1.0
    assert oracle.clip_coefficient(5.0, 0.0) == 1.0


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(1)
    w, g = rng.standard_normal(500), rng.standard_normal(500)
    lr, wd, eps = 1e-3, 0.01, 1e-8
    w1, m1, v1 = oracle.adamw(w, g, np.zeros(500), np.zeros(500), 1, lr, 0.9, 0.999, eps, wd)
    np.testing.assert_allclose(w1, w * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-14, atol=1e-17)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-13)


def test_adamw_constant_gradient_bias_correction_is_exact():
    # With the same gradient at every step, the bias-corrected moments equal g and
    # g^2 exactly, so every step moves w by -lr (g / (|g| + eps) + wd w).
    g = np.array([0.3, -2.0, 1e-3])
    w = np.array([1.0, -0.5, 0.25])
    m = np.zeros(3)
    v = np.zeros(3)
    lr, wd, eps = 0.01, 0.1, 1e-8
    for s in range(1, 8):
        expect = w - lr * (g / (np.abs(g) + eps) + wd * w)
        w, m, v = oracle.adamw(w, g, m, v, s, lr, 0.9, 0.999, eps, wd)
        np.testing.assert_allclose(w, expect, rtol=1e-12)


def test_adamw_gradient_scale_invariance():
    rng = np.random.default_rng(2)
    w, g1, g2 = rng.standard_normal((3, 64))
    a = oracle.adamw(*oracle.adamw(w, g1, 0 * w, 0 * w, 1, 1e-3, 0.9, 0.999, 0.0, 0.01)[:1], g2,
                     *oracle.adamw(w, g1, 0 * w, 0 * w, 1, 1e-3, 0.9, 0.999, 0.0, 0.01)[1:], 2,
                     1e-3, 0.9, 0.999, 0.0, 0.01)[0]
    s = 37.0
    b = oracle.adamw(*oracle.adamw(w, s * g1, 0 * w, 0 * w, 1, 1e-3, 0.9, 0.999, 0.0, 0.01)[:1], s * g2,
                     *oracle.adamw(w, s * g1, 0 * w, 0 * w, 1, 1e-3, 0.9, 0.999, 0.0, 0.01)[1:], 2,
                     1e-3, 0.9, 0.999, 0.0, 0.01)[0]
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_step_applies_clip_before_moments():
    x, t, params, _ = _tiny(16, 4, 6, 3, 2, 6)
    kw = dict(d=4, f=6, E=3, top_k=2)
    free = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, clip_norm=0.0, **kw)
    n = free["grad_norm"]
    clip = n / 10
    clipped = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, clip_norm=clip, **kw)
    c = clip / (n + 1e-6)
    assert clipped["clip_coef"] == pytest.approx(c, rel=1e-15)
    np.testing.assert_allclose(clipped["exp_avg"], 0.1 * c * free["grads"], rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(clipped["exp_avg_sq"], 0.001 * (c * free["grads"]) ** 2, rtol=1e-13, atol=1e-300)


# ----------------------------------------------------------------------------
# Input generator
# ----------------------------------------------------------------------------
def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 3.0e38], np.float32)
    bits = synth.bf16_bits_from_f32(vals)
    back = synth.f32_from_bf16_bits(bits)
    ref = torch.tensor(vals).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, ref)


def test_zipf_bias_fixture_reproduces_target_loads():
    cfg = synth.CONFIGS["zipf_16x8x1024"]
    inp = synth.make_inputs(cfg, 0)
    z = oracle.router_logits(inp.x, inp.w_router, inp.router_bias)
    sel = oracle.token_topk(z, cfg.top_k)
    load = np.bincount(sel.ravel(), minlength=cfg.n_experts) / sel.size
    p = np.arange(1, cfg.n_experts + 1, dtype=np.float64) ** -1.2
    p /= p.sum()
    assert np.abs(load / p - 1).max() <= 0.05


# ----------------------------------------------------------------------------
# Selective updates (router every microbatch, experts on a longer window)
# ----------------------------------------------------------------------------
_SEL = dict(d=6, f=8, E=4, top_k=2, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_selective_step_with_both_groups_is_the_plain_update():
    x, t, params, b = _tiny(40, 6, 8, 4, 2, 21, bias=True)
    m0 = np.abs(np.random.default_rng(1).standard_normal(params.size)) * 1e-3
    v0 = np.abs(np.random.default_rng(2).standard_normal(params.size)) * 1e-6
    plain = oracle.step(x, t, params, m0, v0, 4, clip_norm=0.3, bias=b, **_SEL)
    sel = oracle.selective_step(x, t, params, np.full_like(params, 7.0), m0, v0, step_router=4, step_experts=4,
                                tokens_in_update=40, zero_router=True, zero_experts=True, apply_router=True,
                                apply_experts=True, clip_norm=0.3, bias=b, **_SEL)
    for key in ("params", "exp_avg", "exp_avg_sq", "grads"):
        np.testing.assert_array_equal(sel[key], plain[key])
    assert sel["loss"] == plain["loss"]


def test_selective_router_only_first_step_closed_form():
    # AdamW from zero moments at step 1 moves each weight by lr * (c g / (|c g| + eps) + wd w);
    # the clip norm covers only the router gradient; the experts do not move
    x, t, params, _ = _tiny(32, 6, 8, 4, 2, 22)
    nr = 6 * 4
    g = oracle.step(x, t, params, np.zeros_like(params), np.zeros_like(params), 1, clip_norm=0, **_SEL)["grads"]
    for clip in (0.0, 1e-3):
        out = oracle.selective_step(x, t, params, np.zeros_like(params), np.zeros_like(params),
                                    np.zeros_like(params), step_router=1, step_experts=5, tokens_in_update=32,
                                    zero_router=True, zero_experts=True, apply_router=True, apply_experts=False,
                                    clip_norm=clip, **_SEL)
        gr = g[:nr]
        norm = math.sqrt(float((gr ** 2).sum()))
        assert out["grad_norm"] == pytest.approx(norm, rel=1e-12)
        c = 1.0 if clip == 0 else min(1.0, clip / (norm + 1e-6))
        expect = params[:nr] - _SEL["lr"] * (c * gr / (np.abs(c * gr) + _SEL["eps"]) + _SEL["weight_decay"] * params[:nr])
        np.testing.assert_allclose(out["params"][:nr], expect, rtol=1e-12, atol=1e-15)
        np.testing.assert_array_equal(out["params"][nr:], params[nr:])
        np.testing.assert_array_equal(out["exp_avg"][nr:], 0.0)
        np.testing.assert_allclose(out["grads"], g, rtol=1e-13, atol=1e-17)


def test_selective_expert_window_accumulates_each_microbatch_gradient():
    # router applied every microbatch, experts restarted on the first and applied on
    # the last: the expert gradient used is the sum of the per-microbatch gradients,
    # each taken at the weights in force for that microbatch
    rng = np.random.default_rng(23)
    T, d, f, E, k, n_mb = 24, 6, 8, 4, 2, 3
    xs = [rng.standard_normal((T, d)) for _ in range(n_mb)]
    ts = [rng.standard_normal((T, d)) for _ in range(n_mb)]
    params = np.concatenate([rng.standard_normal(d * E) * 0.8, rng.standard_normal(2 * E * d * f) * 0.5])
    nr = d * E
    p, m, v, grads = params.copy(), np.zeros_like(params), np.zeros_like(params), np.zeros_like(params)
    expert_sum = np.zeros(params.size - nr)
    for i in range(n_mb):
        ref = oracle.step(xs[i], ts[i], p, np.zeros_like(p), np.zeros_like(p), 1, clip_norm=0, **_SEL)["grads"]
        expert_sum += ref[nr:]
        out = oracle.selective_step(xs[i], ts[i], p, grads, m, v, step_router=i + 1, step_experts=1,
                                    tokens_in_update=T, zero_router=True, zero_experts=(i == 0),
                                    apply_router=True, apply_experts=(i == n_mb - 1), clip_norm=0.5, **_SEL)
        np.testing.assert_allclose(out["grads"][:nr], ref[:nr], rtol=1e-12, atol=1e-17)
        np.testing.assert_allclose(out["grads"][nr:], expert_sum, rtol=1e-12, atol=1e-17)
        if i < n_mb - 1:
            np.testing.assert_array_equal(out["params"][nr:], params[nr:])
        p, m, v, grads = out["params"], out["exp_avg"], out["exp_avg_sq"], out["grads"]
    # the experts' single update: AdamW step 1, clipped by the joint norm of the two groups
    # applied in the last launch (the last router gradient and the accumulated expert gradient)
    norm = math.sqrt(float((expert_sum ** 2).sum()) + float((ref[:nr] ** 2).sum()))
    c = min(1.0, 0.5 / (norm + 1e-6))
    w_e, m_e, v_e = oracle.adamw(params[nr:], c * expert_sum, np.zeros_like(expert_sum), np.zeros_like(expert_sum),
                                 1, _SEL["lr"], _SEL["beta1"], _SEL["beta2"], _SEL["eps"], _SEL["weight_decay"])
    np.testing.assert_allclose(p[nr:], w_e, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(v[nr:], v_e, rtol=1e-12, atol=1e-20)
