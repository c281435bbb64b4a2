"""Write the CPU oracle's greedy decode of each workload to greedy_<name>.json.

For each workload: the cache is filled as the workload states (by decoding
its prefill tokens, or with the seeded synthetic prefill), the first decode
token is the first seeded token, and 64 steps follow in which the next token
is the argmax of the oracle's logits (lowest index on ties). Stored per step:
the chosen token and the oracle's top-2 logit margin, so a GPU divergence can
be checked against a near-tie. Calls only oracle/ and synth/.

Usage: python tests/golden/make_greedy.py C1 [C2 ...]
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

STEPS = 64


def greedy_config(name: str):
    """The workload with a decode window of at least STEPS positions."""
    cfg = synth.CONFIGS[name]
    if cfg.steps < STEPS:
        cfg = cfg.with_(steps=STEPS)
    return cfg


def run(name: str) -> dict:
    cfg = greedy_config(name)
    t0 = time.time()
    o = oracle.Oracle.from_config(cfg)
    toks = synth.tokens(cfg)
    if cfg.real_prefill:
        o.prefill_by_decoding(toks[: cfg.ctx])
        first = int(toks[cfg.ctx])
    else:
        first = int(toks[0])
    out, margins = [], []
    t = first
    for s in range(STEPS):
        x = o.step(t, cfg.ctx + s)[-1]
        t, margin = o.greedy(x)
        out.append(t)
        margins.append(margin)
        print(f"{name} step {s}: token {t} margin {margin:.4g} ({time.time() - t0:.0f}s)", flush=True)
    return {"workload": cfg.name, "steps": STEPS, "start_pos": cfg.ctx, "first_token": first,
            "tokens": out, "margins": margins,
            "source": "oracle/ (float64), tests/golden/make_greedy.py"}


if __name__ == "__main__":
    for name in sys.argv[1:]:
        res = run(name)
        with open(os.path.join(HERE, f"greedy_{name}.json"), "w") as f:
            json.dump(res, f, indent=1)
