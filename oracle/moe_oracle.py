"""FP64 CPU oracle for one training update of a top-k mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code with the HIP library.

Everything is plain float64 NumPy with one matrix product per expert; there is
no blocking, fusion or reordering beyond the definitions below, so each line can
be checked against the pages by eye.  Sources (Latch project pages):

* "How a training megakernel works", section "One training update": the chain
  rule, the squared-error loss L = 1/2 (y - t)^2 and the plain SGD step of the
  two-weight example (used here for the worked-example pin).
* same page, "From two weights to 200 million": each expert layer of the
  pages' model routes every token to 2 of its 16 expert feed-forward blocks, and
  the optimizer is AdamW (exponential moving averages of the gradient and of its
  elementwise square).
* same page, "What Latch does", step 1: the layer is expressed with the routing
  and grouped-product operations ``token_topk``, ``route_order`` and
  ``ragged_mm``; clipping by the global gradient norm and the AdamW step are
  ordinary tensor expressions handed to the update rule.
* same page, step 3: each expert's gradient has to flow back to the tokens that
  were sent to that expert.
* same page, step 4: master weights and both Adam moments are stored in FP32
  (the storage the oracle reads; it computes in float64).

The pages do not write the layer's formulas.  The readings adopted where they are
silent:

* layer output y_i = sum_j g_ij * FFN_{e_ij}(x_i); FFN_e(x) = gelu(x W1[e]) W2[e];
  no biases, residual, norm or auxiliary loss; the skewed-load workload adds a
  constant (untrained) router bias;
* top-k order: descending logit, the lower expert index wins a tie (+0 and -0 tie);
* gates: softmax over the k selected logits only;
* no gradient flows through the choice of experts, only through the gates;
* route_order: stable by expert, so inside an expert rows ascend by flat id i*k+j;
* loss L = sum_i ||y_i - t_i||^2 / (2 * T_update), T_update = tokens in the update;
* GELU in its tanh form; clipping c = min(1, clip / (||g|| + 1e-6)) over all
  parameters jointly, before the moments; AdamW with decoupled decay on every
  parameter, eps outside the square root, bias correction with the 1-based step.
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715
CLIP_EPS = 1e-6


# ----------------------------------------------------------------------------
# Elementwise functions
# ----------------------------------------------------------------------------
def gelu_tanh(h):
    """GELU, tanh form: 1/2 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3)))."""
    h = np.asarray(h, dtype=np.float64)
    u = SQRT_2_OVER_PI * (h + GELU_CUBIC * h ** 3)
    return 0.5 * h * (1.0 + np.tanh(u))


def gelu_tanh_grad(h):
    """Derivative of ``gelu_tanh`` with respect to h."""
    h = np.asarray(h, dtype=np.float64)
    u = SQRT_2_OVER_PI * (h + GELU_CUBIC * h ** 3)
    th = np.tanh(u)
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * h ** 2)
    return 0.5 * (1.0 + th) + 0.5 * h * (1.0 - th ** 2) * du


def _identity(h):
    return np.asarray(h, dtype=np.float64)


def _identity_grad(h):
    return np.ones_like(np.asarray(h, dtype=np.float64))


ACTIVATIONS = {"gelu_tanh": (gelu_tanh, gelu_tanh_grad), "identity": (_identity, _identity_grad)}


# ----------------------------------------------------------------------------
# Routing: router logits, token_topk, route_order ("What Latch does", step 1)
# ----------------------------------------------------------------------------
def router_logits(x, w_router, bias=None):
    """z = x W_r (+ b): one logit per (token, expert)."""
    z = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)
    if bias is not None:
        z = z + np.asarray(bias, np.float64)[None, :]
    return z


def token_topk(z, k):
    """Per token, the k experts with the largest logits, largest first; on equal
    logits the lower expert index comes first.  Returns int64 [T, k].

    A stable sort of -z keeps equal keys in ascending index order, which is the
    tie rule.  +0.0 and -0.0 compare equal and so tie.  NaN logits are rejected.
    """
    z = np.asarray(z)
    if np.isnan(z).any():
        raise ValueError("token_topk: NaN router logit")
    order = np.argsort(-z, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_gates(z, sel):
    """Softmax over the k selected logits of each token (max subtracted)."""
    zs = np.take_along_axis(np.asarray(z, np.float64), sel, axis=1)
    zs = zs - zs.max(axis=1, keepdims=True)
    ez = np.exp(zs)
    return ez / ez.sum(axis=1, keepdims=True)


def route_order(sel, n_experts):
    """Stable bucketing of the flat routed ids q = i*k + j by expert.

    Returns (counts[E], offsets[E+1], perm[N], inv[N]): ``perm[p]`` is the flat id
    at sorted position p; ``inv[q]`` is the position of flat id q.
    """
    keys = np.asarray(sel).reshape(-1)
    perm = np.argsort(keys, kind="stable").astype(np.int64)
    counts = np.bincount(keys, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int64)
    return counts, offsets, perm, inv


# ----------------------------------------------------------------------------
# Forward, loss, backward of the layer
# ----------------------------------------------------------------------------
def layer_forward(x, t, w_router, w1, w2, top_k, tokens_in_update, *, bias=None,
                  act="gelu_tanh", forced_topk=None):
    """Forward pass and loss.  Returns a dict of every intermediate the backward
    pass reads (the values the example's backward "reads from the forward pass")."""
    x = np.asarray(x, np.float64)
    t = np.asarray(t, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    T, d = x.shape
    E = w1.shape[0]
    f = w1.shape[2]
    k = top_k
    fn, _ = ACTIVATIONS[act]

    z = router_logits(x, w_router, bias)
    sel = token_topk(z, k) if forced_topk is None else np.asarray(forced_topk, np.int64).reshape(T, k)
    g = topk_gates(z, sel)
    counts, offsets, perm, inv = route_order(sel, E)

    N = T * k
    rows = perm // k                      # token of each sorted position
    H = np.zeros((N, f))
    A = np.zeros((N, f))
    O = np.zeros((N, d))
    for e in range(E):
        seg = slice(offsets[e], offsets[e + 1])
        Xe = x[rows[seg]]                 # dispatch gather
        H[seg] = Xe @ w1[e]               # ragged_mm, first product
        A[seg] = fn(H[seg])
        O[seg] = A[seg] @ w2[e]           # ragged_mm, second product

    Og = O[inv].reshape(T, k, d)          # expert outputs in (token, slot) order
    y = np.einsum("tk,tkd->td", g, Og)    # weighted combine
    r = y - t
    loss = float((r * r).sum() / (2.0 * tokens_in_update))
    return dict(x=x, t=t, z=z, sel=sel, g=g, counts=counts, offsets=offsets, perm=perm,
                inv=inv, rows=rows, H=H, A=A, O=O, y=y, loss=loss, k=k, E=E,
                tokens_in_update=tokens_in_update, act=act)


def layer_backward(fw, w_router, w1, w2):
    """Chain rule through the layer.  Returns (dW_r, dW1, dW2, dx)."""
    x, t, g, sel, inv, rows, offsets = fw["x"], fw["t"], fw["g"], fw["sel"], fw["inv"], fw["rows"], fw["offsets"]
    H, A, O, y = fw["H"], fw["A"], fw["O"], fw["y"]
    k, E = fw["k"], fw["E"]
    T, d = x.shape
    w_router = np.asarray(w_router, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    _, dfn = ACTIVATIONS[fw["act"]]

    dy = (y - t) / fw["tokens_in_update"]                     # dL/dy
    Og = O[inv].reshape(T, k, d)
    dg = np.einsum("td,tkd->tk", dy, Og)                      # dL/dg
    dOg = g[:, :, None] * dy[:, None, :]                      # dL/dO in (token, slot) order
    dO = np.empty_like(O)
    dO[inv] = dOg.reshape(T * k, d)                           # back to sorted positions

    # softmax over the selected logits: dz_j = g_j (dg_j - sum_l g_l dg_l)
    dzs = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    dz = np.zeros((T, E))
    np.put_along_axis(dz, sel, dzs, axis=1)
    dW_r = x.T @ dz
    dx = dz @ w_router.T

    dW1 = np.zeros_like(w1)
    dW2 = np.zeros_like(w2)
    dXs = np.zeros((T * k, d))
    for e in range(E):
        seg = slice(offsets[e], offsets[e + 1])
        Xe = x[rows[seg]]
        dA = dO[seg] @ w2[e].T
        dW2[e] = A[seg].T @ dO[seg]
        dH = dA * dfn(H[seg])
        dW1[e] = Xe.T @ dH
        dXs[seg] = dH @ w1[e].T
    # gradient back to tokens: each token receives exactly its k contributions
    dx = dx + dXs[inv].reshape(T, k, d).sum(axis=1)
    return dW_r, dW1, dW2, dx


# ----------------------------------------------------------------------------
# Optimizer: global-norm clipping and AdamW (step 1 of "What Latch does")
# ----------------------------------------------------------------------------
def global_norm(grads):
    return math.sqrt(sum(float((np.asarray(g, np.float64) ** 2).sum()) for g in grads))


def clip_coefficient(norm, clip_norm):
    """c = min(1, clip / (norm + 1e-6)); clip_norm <= 0 disables clipping."""
    if clip_norm <= 0:
        return 1.0
    return min(1.0, clip_norm / (norm + CLIP_EPS))


def adamw(w, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """One AdamW update of flat arrays (returns new w, m, v; inputs untouched)."""
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    w_new = w - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * w)
    return w_new, m, v


def sgd(w, g, lr):
    """Plain gradient step, as in the two-weight example."""
    return np.asarray(w, np.float64) - lr * np.asarray(g, np.float64)


# ----------------------------------------------------------------------------
# One complete update
# ----------------------------------------------------------------------------
def unpack_params(flat, d, f, E):
    flat = np.asarray(flat, np.float64)
    n_r, n_1 = d * E, E * d * f
    return (flat[:n_r].reshape(d, E), flat[n_r:n_r + n_1].reshape(E, d, f),
            flat[n_r + n_1:n_r + 2 * n_1].reshape(E, f, d))


def pack(w_r, w1, w2):
    return np.concatenate([np.ravel(w_r), np.ravel(w1), np.ravel(w2)]).astype(np.float64)


def step(xs, ts, params, exp_avg, exp_avg_sq, step_index, *, d, f, E, top_k,
         lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, clip_norm=1.0,
         bias=None, act="gelu_tanh", opt="adamw", forced_topk=None, with_loss_after=False):
    """One training update over one or more microbatches.

    ``xs``/``ts`` are lists of [T_m, d] arrays (one per microbatch; gradients are
    summed across them in float64 and the loss is the mean over all their
    tokens).  ``params``/``exp_avg``/``exp_avg_sq`` are flat vectors in the order
    W_r | W1 | W2.  ``forced_topk`` (list, one [T_m, k] per microbatch) replaces the
    selection, for comparing against a GPU's own routing.
    """
    if isinstance(xs, np.ndarray):
        xs, ts = [xs], [ts]
        if forced_topk is not None:
            forced_topk = [forced_topk]
    w_r, w1, w2 = unpack_params(params, d, f, E)
    t_upd = sum(int(np.shape(x)[0]) for x in xs)

    loss = 0.0
    gr = np.zeros_like(w_r)
    g1 = np.zeros_like(w1)
    g2 = np.zeros_like(w2)
    dxs, routing = [], []
    for i, (x, t) in enumerate(zip(xs, ts)):
        fw = layer_forward(x, t, w_r, w1, w2, top_k, t_upd, bias=bias, act=act,
                           forced_topk=None if forced_topk is None else forced_topk[i])
        dgr, dg1, dg2, dx = layer_backward(fw, w_r, w1, w2)
        loss += fw["loss"]
        gr += dgr
        g1 += dg1
        g2 += dg2
        dxs.append(dx)
        routing.append({key: fw[key] for key in ("z", "sel", "g", "counts", "offsets", "perm", "inv")})

    grads = pack(gr, g1, g2)
    norm = global_norm([grads])
    if opt == "adamw":
        c = clip_coefficient(norm, clip_norm)
        new_p, new_m, new_v = adamw(params, c * grads, exp_avg, exp_avg_sq, step_index,
                                    lr, beta1, beta2, eps, weight_decay)
    elif opt == "sgd":
        c = clip_coefficient(norm, clip_norm)
        new_p = sgd(params, c * grads, lr)
        new_m = np.asarray(exp_avg, np.float64)
        new_v = np.asarray(exp_avg_sq, np.float64)
    else:
        raise ValueError(opt)

    out = dict(loss=loss, grads=grads, grad_norm=norm, clip_coef=c, params=new_p,
               exp_avg=new_m, exp_avg_sq=new_v, dx=dxs if len(dxs) > 1 else dxs[0],
               routing=routing if len(routing) > 1 else routing[0])
    if with_loss_after:
        nr, n1, n2 = unpack_params(new_p, d, f, E)
        out["loss_after"] = sum(layer_forward(x, t, nr, n1, n2, top_k, t_upd, bias=bias, act=act)["loss"]
                                for x, t in zip(xs, ts))
    return out


def selective_step(x, t, params, grads, exp_avg, exp_avg_sq, *, step_router, step_experts, d, f, E, top_k,
                   tokens_in_update, zero_router, zero_experts, apply_router, apply_experts,
                   lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, clip_norm=1.0,
                   bias=None, act="gelu_tanh", forced_topk=None):
    """One microbatch of the selective-update scheme (Latch pages, "Results",
    table "Other measured compiler work": the shared weights update every
    microbatch, the experts every 16).  Two parameter groups, the router W_r and
    the experts W1 | W2, each with its own gradient accumulation window and its
    own AdamW step count.

    The pages give only the schedule; the reading taken here: the microbatch's
    gradient (loss denominator ``tokens_in_update``) is added to the running
    gradient of each group, which first restarts from zero for a group whose
    ``zero_*`` flag is set; each group whose ``apply_*`` flag is set then gets
    global-norm clipping and AdamW, the norm taken over the applied groups'
    running gradients jointly (with both applied this is exactly ``step``).
    Groups not applied keep their weights and moments.  Returns the new
    params / grads / moments, the loss, dx and the routing."""
    w_r, w1, w2 = unpack_params(params, d, f, E)
    fw = layer_forward(x, t, w_r, w1, w2, top_k, tokens_in_update, bias=bias, act=act, forced_topk=forced_topk)
    dgr, dg1, dg2, dx = layer_backward(fw, w_r, w1, w2)
    nr = d * E
    g_old = np.asarray(grads, np.float64)
    g_new = pack(dgr, dg1, dg2)
    acc = g_new.copy()
    if not zero_router:
        acc[:nr] += g_old[:nr]
    if not zero_experts:
        acc[nr:] += g_old[nr:]
    new_p = np.asarray(params, np.float64).copy()
    new_m = np.asarray(exp_avg, np.float64).copy()
    new_v = np.asarray(exp_avg_sq, np.float64).copy()
    applied = [s for s, on in ((slice(0, nr), apply_router), (slice(nr, None), apply_experts)) if on]
    norm, c = None, None
    if applied:
        norm = global_norm([acc[s] for s in applied])
        c = clip_coefficient(norm, clip_norm)
        for s, on, stp in ((slice(0, nr), apply_router, step_router), (slice(nr, None), apply_experts, step_experts)):
            if on:
                new_p[s], new_m[s], new_v[s] = adamw(new_p[s], c * acc[s], new_m[s], new_v[s], stp,
                                                     lr, beta1, beta2, eps, weight_decay)
    return dict(loss=fw["loss"], grads=acc, grad_norm=norm, clip_coef=c, params=new_p, exp_avg=new_m,
                exp_avg_sq=new_v, dx=dx,
                routing={key: fw[key] for key in ("z", "sel", "g", "counts", "offsets", "perm", "inv")})


def forward_loss(x, t, params, *, d, f, E, top_k, bias=None, act="gelu_tanh", forced_topk=None,
                 tokens_in_update=None):
    """Loss only (used by finite-difference pins)."""
    w_r, w1, w2 = unpack_params(params, d, f, E)
    tu = np.shape(x)[0] if tokens_in_update is None else tokens_in_update
    return layer_forward(x, t, w_r, w1, w2, top_k, tu, bias=bias, act=act, forced_topk=forced_topk)["loss"]
