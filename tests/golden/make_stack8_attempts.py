"""Writes stack8_attempts.json: the draw attempt of every token of the
8-layer + int8 draft stack workload such that, at every layer of the oracle's
chain, no token has two of its k+1 best router scores closer than 1e-6.

Calls only the seeded input generator and the CPU oracle. Run from the
repository root:  python tests/golden/make_stack8_attempts.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from tests import layer_cases as lc  # noqa: E402


def main():
    cfg = synth.CONFIGS["stack8_draft"]
    attempts = np.zeros(cfg.n_tokens, np.int64)
    todo = np.arange(cfg.n_tokens)
    rounds = 0
    t0 = time.time()
    while len(todo):
        rounds += 1
        bad = lc.stack_chain(cfg, attempts, tokens=todo)
        bad_tokens = todo[bad]
        print(f"round {rounds}: {len(todo)} tokens run, {len(bad_tokens)} redrawn "
              f"({time.time() - t0:.0f}s)", flush=True)
        attempts[bad_tokens] += 1
        todo = bad_tokens
    out = {
        "source": "tests/golden/make_stack8_attempts.py (seeded generator + CPU oracle only)",
        "config": cfg.name,
        "gap": lc.GAP,
        "attempts": attempts.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stack8_attempts.json")
    with open(path, "w") as fh:
        json.dump(out, fh)
    print(f"wrote {path}: {int((attempts > 0).sum())} tokens redrawn in {rounds} rounds")


if __name__ == "__main__":
    main()
