"""moe_layer_step (route, union, count and the expert step in one call)
against moe_route_union + moe_expert_forward on the same inputs, bit for bit,
and against the oracle.

One or two tokens take the routing inside the gate/up GEMV launch; larger
batches take the two calls' kernels. Counters must accumulate as with the two calls.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import int4_routed_expert_gemv_amd as moe
import oracle
import synth
from tests import layer_cases as lc
from tests.gpu_layer import run_layer, run_layer_step, upload_pool

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _compare(cfg, shared=True, dup=False):
    spec = cfg.layers[0]
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    if dup:
        # every token a copy of token 0 (each token's gaps stay clear): all
        # tokens pick the same experts, so each routed item holds every token
        x = np.ascontiguousarray(np.broadcast_to(x[:1], x.shape))
    blocks, sh = lc.canonical_pool(cfg, 0)
    if not shared:
        sh = None
    say(f"[layer_step] {cfg.name} N={cfg.n_tokens} k={cfg.k} d={spec.d} f={spec.f} "
        f"E={spec.n_experts} wbits={spec.wbits} shared={shared} dup={dup}")
    ref = oracle.layer_step(x, wr, b, cfg.k, blocks, sh, spec.d, spec.f, spec.wbits, spec.group)
    pool = upload_pool(spec, blocks, sh)
    two = run_layer(pool, x, wr, b, cfg.k, fused_route=True)
    one = run_layer_step(pool, x, wr, b, cfg.k)
    for key in ("ids", "w", "union_ids", "offsets", "perm", "counters", "y"):
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    assert one["n_union"] == two["n_union"]
    np.testing.assert_array_equal(one["ids"], ref["ids"])
    np.testing.assert_array_equal(one["union_ids"], ref["union_ids"])
    np.testing.assert_array_equal(one["perm"], ref["perm"])
    np.testing.assert_array_equal(one["counters"], ref["counters"])
    np.testing.assert_array_equal(one["offsets"], ref["offsets"])
    if dup:
        assert len(ref["union_ids"]) == cfg.k and np.all(ref["counters"][ref["union_ids"]] ==
                                                          cfg.n_tokens)
    err = lc.rel_err_rows(one["y"], ref["y"]).max()
    assert err <= 2e-3, f"max per-token relative error {err:.3e}"
    # counters accumulate over calls
    again = run_layer_step(pool, x, wr, b, cfg.k, counters=one["counters_t"])
    np.testing.assert_array_equal(again["counters"], 2 * ref["counters"])
    np.testing.assert_array_equal(again["y"], one["y"])
    say(f"[layer_step] equal to the two calls, max rel err {err:.2e}")
    del pool
    torch.cuda.empty_cache()


def test_decode1():
    _compare(synth.CONFIGS["decode1"])


@pytest.mark.parametrize("k", [2, 8])
def test_decode_shapes_one_token_topk(k):
    _compare(dataclasses.replace(synth.CONFIGS["decode1"], k=k))


@pytest.mark.parametrize("k", [1, 8])
def test_decode_shapes_two_tokens(k):
    """A two-token verify batch on the decode layer's shapes (Zipf router
    bias, so the two tokens share experts): routing inside the gate/up
    launch with items of one and two tokens."""
    _compare(dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=2, k=k))


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("name", ["decode64", "tiny"])
@pytest.mark.parametrize("shared", [True, False])
def test_two_tokens_same_experts(name, k, shared):
    """Two identical tokens: the in-launch routing of one or two tokens meets
    a routed expert that holds both of them (items of two tokens, the second
    token found at permutation position 1, a hit count of 2 per expert)."""
    _compare(dataclasses.replace(synth.CONFIGS[name], n_tokens=2, k=k), shared=shared, dup=True)


@pytest.mark.parametrize("N,k,shared", [(1, 1, True), (1, 1, False), (1, 2, False), (1, 5, True),
                                        (1, 16, True), (2, 1, True), (2, 1, False), (2, 2, False),
                                        (2, 3, True), (2, 8, True), (2, 16, False), (3, 2, True),
                                        (4, 8, True), (40, 4, True)])
def test_tiny(N, k, shared):
    _compare(dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=N, k=k), shared=shared)


@pytest.mark.parametrize("E,k,N", [(1000, 32, 1), (1024, 7, 1), (65, 3, 1), (1000, 32, 2),
                                   (65, 5, 2)])
def test_one_token_many_experts(E, k, N):
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=N, k=k,
                              layers=(dataclasses.replace(base.layer, n_experts=E),))
    _compare(cfg)


@pytest.mark.parametrize("N", [1, 2])
def test_one_token_int8(N):
    base = synth.CONFIGS["tiny"]
    spec = dataclasses.replace(base.layer, wbits=8, group=0, scale_lo=0.005 / 16,
                               scale_hi=0.02 / 16)
    _compare(dataclasses.replace(base, n_tokens=N, k=3, layers=(spec,)))


@pytest.mark.parametrize("big,small", [(1, -1), (-1, 1), (-1, -1)])
def test_one_token_with_thresholds(big, small):
    """Options: a positive threshold puts the one token on a matrix-core pass
    (the two calls' kernels), -1 on both keeps the routing inside the gate/up
    launch; each equals moe_expert_forward_ex with the same thresholds."""
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=1, k=3)
    spec = cfg.layers[0]
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    blocks, sh = lc.canonical_pool(cfg, 0)
    say(f"[layer_step] thresholds big={big} small={small}")
    ref = oracle.layer_step(x, wr, b, cfg.k, blocks, sh, spec.d, spec.f, spec.wbits, spec.group)
    pool = upload_pool(spec, blocks, sh)
    opts = moe.ForwardOptions()
    opts.mfma_min_tokens = big
    opts.mfma_small_min_tokens = small
    one = run_layer_step(pool, x, wr, b, cfg.k, options=opts)
    two = run_layer(pool, x, wr, b, cfg.k, fused_route=True, mfma_min_tokens=big,
                    mfma_small_min_tokens=small)
    for key in ("ids", "w", "union_ids", "offsets", "perm", "counters", "y"):
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    np.testing.assert_array_equal(one["ids"], ref["ids"])
    assert lc.rel_err_rows(one["y"], ref["y"]).max() <= 2e-3
    del pool
    torch.cuda.empty_cache()
