"""Writes the oracle regression snapshot; calls only oracle/ and the seeded input generator."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from mixture_experts_layer_30_amd import configs, synth  # noqa: E402


def main():
    s = configs.CONFIGS["tiny"]
    d = synth.layer_inputs(s, 64, dense=False)
    out, ids, w = oracle.moe_layer(d["x"], d["logits"], d["w13"], d["w2"], s.topk)
    np.savez(os.path.join(HERE, "oracle_tiny_T64.npz"), x=d["x"].numpy(), ids=ids, w=w, out=out)


if __name__ == "__main__":
    main()
