"""Seeded synthetic inputs for one MoE-layer training update.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the FP64 oracle (through the tests) and the HIP path
(through the tests, ``bench.py`` and ``__graft_entry__.smoke``) read the same
arrays from here, so the two implementations see bit-identical inputs.

Recipe (Latch "How a training megakernel works": in "From two weights to 200
million" each expert layer routes a token to 2 of 16 expert feed-forward blocks;
the batch shapes 2x1024, 32x1024 and 16 x 8x1024 come from the same page's
"Many small routed experts" section and the results table):

* ``numpy.random.default_rng(seed)`` draws, in this order and as float64
  standard normals: x [T,d], t [T,d], W_r [d,E], W1 [E,d,f], W2 [E,f,d].
  Activations and targets are N(0,1); weights are N(0, 0.02^2) (0.02 is the
  standard deviation).  Everything is cast to fp32.  In bf16 mode x and t are
  then rounded to bf16 (round to nearest, ties to even) and both sides read
  those bf16 values.
* Adam moments start at zero.
* The skewed-load case adds a constant router bias read from
  ``tests/golden/zipf_bias_s1p2.json`` (written by the committed calibration
  script next to it).
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_GOLDEN = os.path.join(os.path.dirname(_HERE), "tests", "golden")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and hyper-parameters of one MoE feed-forward layer update."""
    name: str
    tokens: int          # tokens in one launch (one microbatch)
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    dtype: str           # "f32" or "bf16"
    microbatches: int = 1
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    clip_norm: float = 1.0
    zipf_bias: bool = False

    @property
    def tokens_in_update(self) -> int:
        return self.tokens * self.microbatches

    @property
    def param_count(self) -> int:
        d, f, e = self.d_model, self.d_ff, self.n_experts
        return d * e + 2 * e * d * f


# The five workloads.  C0 is small enough for the oracle in well under a second.
CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", 256, 64, 128, 4, 2, "f32"),
    "bf16_2x1024": LayerConfig("bf16_2x1024", 2 * 1024, 768, 1536, 16, 2, "bf16"),
    "bf16_32x1024": LayerConfig("bf16_32x1024", 32 * 1024, 768, 1536, 16, 2, "bf16"),
    "zipf_16x8x1024": LayerConfig("zipf_16x8x1024", 8 * 1024, 768, 1536, 16, 2, "bf16",
                                  microbatches=16, zipf_bias=True),
    "top8_4x1024": LayerConfig("top8_4x1024", 4 * 1024, 1024, 512, 64, 8, "bf16"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (at most
    # 0xFF800000 + 0x8000); NaNs are replaced below
    out = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class LayerInputs:
    """Host copies of every input.  ``x``/``t`` are fp32 arrays holding exactly the
    stored values (bf16-representable in bf16 mode); ``x_bits``/``t_bits`` are the
    uint16 bf16 patterns in bf16 mode (None in f32 mode)."""
    cfg: LayerConfig
    x: np.ndarray            # [microbatches*T, d] float32
    t: np.ndarray            # [microbatches*T, d] float32
    w_router: np.ndarray     # [d, E] float32
    w1: np.ndarray           # [E, d, f] float32
    w2: np.ndarray           # [E, f, d] float32
    router_bias: np.ndarray | None   # [E] float32 or None
    x_bits: np.ndarray | None = None
    t_bits: np.ndarray | None = None

    def flat_params(self) -> np.ndarray:
        """Flat fp32 parameter vector in the library's order: W_r | W1 | W2."""
        return np.concatenate([self.w_router.ravel(), self.w1.ravel(), self.w2.ravel()]).astype(np.float32)

    def microbatch(self, i: int):
        T = self.cfg.tokens
        sl = slice(i * T, (i + 1) * T)
        return self.x[sl], self.t[sl]


def zipf_bias(cfg: LayerConfig) -> np.ndarray:
    """Constant router bias for the Zipf(1.2) skewed-load workload, read from the
    stored fixture (calibrated against the oracle's routing by
    ``tests/golden/make_zipf_bias.py``)."""
    path = os.path.join(_GOLDEN, "zipf_bias_s1p2.json")
    with open(path) as fh:
        doc = json.load(fh)
    key = f"{cfg.tokens}x{cfg.microbatches}_d{cfg.d_model}_E{cfg.n_experts}_k{cfg.top_k}_seed{doc['seed']}"
    if key not in doc["bias"]:
        raise KeyError(f"no calibrated Zipf bias stored for {key}")
    return np.asarray(doc["bias"][key], dtype=np.float32)


def make_inputs(cfg: LayerConfig, seed: int = 0, *, with_bias: bool | None = None) -> LayerInputs:
    """Draw the inputs of ``cfg`` from ``default_rng(seed)`` in the documented order."""
    rng = np.random.default_rng(seed)
    T = cfg.tokens * cfg.microbatches
    d, f, E = cfg.d_model, cfg.d_ff, cfg.n_experts
    x = rng.standard_normal((T, d)).astype(np.float32)
    t = rng.standard_normal((T, d)).astype(np.float32)
    w_r = (0.02 * rng.standard_normal((d, E))).astype(np.float32)
    w1 = (0.02 * rng.standard_normal((E, d, f))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((E, f, d))).astype(np.float32)
    x_bits = t_bits = None
    if cfg.dtype == "bf16":
        x_bits = bf16_bits_from_f32(x)
        t_bits = bf16_bits_from_f32(t)
        x = f32_from_bf16_bits(x_bits)
        t = f32_from_bf16_bits(t_bits)
    use_bias = cfg.zipf_bias if with_bias is None else with_bias
    bias = zipf_bias(cfg) if use_bias else None
    return LayerInputs(cfg, x, t, w_r, w1, w2, bias, x_bits, t_bits)


def small_config(name="tiny", tokens=256, d=64, f=128, E=4, k=2, dtype="f32", **kw) -> LayerConfig:
    """A custom-sized config for parity cases (ragged tails, odd sizes)."""
    return LayerConfig(name, tokens, d, f, E, k, dtype, **kw)
