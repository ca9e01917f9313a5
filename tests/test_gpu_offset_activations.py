"""Layer outputs when every activation carries a large common offset.

On the 32-token pass of int4 layers whose scale groups cover whole 128-column
unit steps, the gate/up kernel feeds the matrix cores codes that still carry
their float16 bias (1032 + q, or 1152 + 16 q against an activation divided by
16) and takes the biases out with a separate chain of products per token
block, added to each unit step's float32 sums before they are scaled. The
float32 rounding of those two sums grows with the activations' sum over the
step, so the worst case is activations that all share one sign and a large
mean. Here x = mu + N(0, 1) with mu up to 16, on a layer with groups of 128,
routed by a zero router with stepped biases (every token takes the same
top-2 experts, so each holds all 64 tokens and both it and the shared expert
run on the 32-token pass). Outputs must still match the oracle's to the usual
2e-3 per token, and the routing bit for bit.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import layer_cases as lc
from tests.gpu_layer import run_layer, upload_pool

pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def offset_config(n_tokens=64, k=2):
    spec = synth.LayerSpec(d=1024, f=512, n_experts=16, wbits=4, group=128,
                           scale_lo=0.005, scale_hi=0.02, bias="zero")
    return dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=n_tokens, k=k, layers=(spec,))


@pytest.mark.parametrize("mu", [0.0, 4.0, 16.0, -16.0])
def test_offset_activations_small_pass(mu):
    cfg = offset_config()
    spec = cfg.layer
    E, d, k = spec.n_experts, spec.d, cfg.k
    # zero router, biases rising in steps of 0.01: experts E-1 and E-2 win
    # for every token, whatever x holds
    wr = np.zeros((E, d), np.float32)
    b = (0.01 * np.arange(E)).astype(np.float32)
    x = (synth.tokens(cfg) + np.float32(mu)).astype(np.float32)
    blocks, shared = lc.canonical_pool(cfg)
    say(f"[offset] mu={mu} N={cfg.n_tokens} k={k} d={d} f={spec.f} G={spec.group}")
    ref = oracle.layer_step(x, wr, b, k, blocks, shared, d, spec.f, spec.wbits, spec.group)
    np.testing.assert_array_equal(ref["ids"], np.tile([E - 1, E - 2], (cfg.n_tokens, 1)))
    pool = upload_pool(spec, blocks, shared)   # packs the blocks in place: oracle first
    got = run_layer(pool, x, wr, b, k)
    for key in ("ids", "union_ids", "offsets", "perm", "counters"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    err = lc.rel_err_rows(got["y"], ref["y"])
    say(f"[offset] mu={mu}: max per-token relative error {err.max():.2e}")
    assert np.all(np.isfinite(got["y"]))
    assert err.max() <= TOL, f"max per-token relative error {err.max():.3e} > {TOL}"
