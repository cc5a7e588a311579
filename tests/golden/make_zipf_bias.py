"""Write ``zipf_bias_s1p2.json``: the constant router bias of the skewed-load
workload (16 microbatches of 8x1024 tokens, d=768, 16 experts, top-2).

Target expert loads follow Zipf with exponent 1.2: p_e proportional to
(e+1)^-1.2, expert 0 heaviest.  The bias starts at ln p and is corrected by a
fraction (first 1/2, halved whenever the error grows) of the log-ratio between
target and realised top-2 load, measured over all 16 microbatches with the
oracle's own routing (FP64 logits), until every expert's load is within 5% of
its target.  Only ``oracle/`` and the seeded input
generator are called.

Run from the repository root:  python tests/golden/make_zipf_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

SEED = 0


def main():
    cfg = synth.CONFIGS["zipf_16x8x1024"]
    inp = synth.make_inputs(cfg, SEED, with_bias=False)
    E, k = cfg.n_experts, cfg.top_k
    p = (np.arange(1, E + 1, dtype=np.float64)) ** -1.2
    p /= p.sum()
    z0 = oracle.router_logits(inp.x, inp.w_router)
    b = np.log(p)
    alpha, prev = 0.5, np.inf
    for it in range(400):
        sel = oracle.token_topk(z0 + b.astype(np.float32).astype(np.float64)[None, :], k)
        load = np.bincount(sel.ravel(), minlength=E) / sel.size
        err = np.abs(load / p - 1.0).max()
        print(f"iter {it}: max relative load error {err:.4f}")
        if err <= 0.05:
            break
        if err > prev:
            alpha *= 0.5
        prev = err
        b = b + alpha * (np.log(p) - np.log(np.maximum(load, 1e-9)))
    else:
        raise SystemExit("calibration did not converge")
    key = f"{cfg.tokens}x{cfg.microbatches}_d{cfg.d_model}_E{E}_k{k}_seed{SEED}"
    doc = {
        "what": "constant router bias for the Zipf(s=1.2) skewed-load workload",
        "written_by": "tests/golden/make_zipf_bias.py (oracle routing only)",
        "seed": SEED,
        "zipf_exponent": 1.2,
        "target_load": p.tolist(),
        "realised_load": load.tolist(),
        "bias": {key: b.astype(np.float32).astype(float).tolist()},
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_s1p2.json")
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
