"""Writes the seeded inputs of one workload to a binary file that the C++
driver of the C ABI (``moe_step_bench --inputs FILE``) reads, so profiled
launches see exactly the inputs the tests and ``bench.py`` use.

    python -m synth.dump --config NAME [--seed S] --out FILE

Layout (little endian): 8-byte magic ``MOEIN001``; int32 tokens per launch,
microbatches, d_model, d_ff, n_experts, top_k, dtype (0 fp32, 1 bf16),
has_bias; then x [microbatches * tokens, d] and t (bf16 bit patterns or fp32),
the flat fp32 parameters W_r | W1 | W2, and the fp32 router bias [E] when
has_bias is 1."""
from __future__ import annotations

import argparse
import struct

import numpy as np

from . import CONFIGS, make_inputs

MAGIC = b"MOEIN001"


def dump(cfg, seed: int, path: str) -> None:
    inp = make_inputs(cfg, seed)
    bf16 = cfg.dtype == "bf16"
    has_bias = inp.router_bias is not None
    with open(path, "wb") as fh:
        fh.write(MAGIC)
        fh.write(struct.pack("<8i", cfg.tokens, cfg.microbatches, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k,
                             1 if bf16 else 0, 1 if has_bias else 0))
        for arr, bits in ((inp.x, inp.x_bits), (inp.t, inp.t_bits)):
            data = np.ascontiguousarray(bits, dtype="<u2") if bf16 else np.ascontiguousarray(arr, dtype="<f4")
            fh.write(data.tobytes())
        fh.write(np.ascontiguousarray(inp.flat_params(), dtype="<f4").tobytes())
        if has_bias:
            fh.write(np.ascontiguousarray(inp.router_bias, dtype="<f4").tobytes())


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--config", required=True, choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    dump(CONFIGS[args.config], args.seed, args.out)
    print(f"wrote {args.out}")


if __name__ == "__main__":
    main()
