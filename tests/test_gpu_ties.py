"""Exact score ties on the GPU: the lowest expert id wins, on every route path.

The top-k ranks experts by float32 score and breaks ties toward the lower
expert id ("ties broken by lowest index"). The other parity tests redraw any
token whose best scores lie within 1e-6 of each other, so they never meet a
tie. Here ties are built on purpose, in three ways:

  pairs  router rows and biases duplicated in pairs (expert 2i+1 is a copy of
         expert 2i): every score has an exact twin, so an odd k takes the
         lower id of a pair and leaves its twin out; only the gaps between
         distinct pairs follow the 1e-6 redraw rule;
  zero   a zero router with zero bias: every score is exactly 0.5 and every
         token routes to experts 0 .. k-1;
  steps  a zero router whose bias rises in groups of four equal values, 0.01
         apart (scores about 2.5e-3 apart, far above the 1e-6 redraw gap):
         the best group first, its four ids ascending, then the next group.

Each case runs at 1, 2, 16, 17, 64 and 4096 tokens, so that every route path
is taken: the in-GEMV routing of moe_layer_step (one or two tokens, top-1 or
top-2), the one-workgroup route tail (up to 16 tokens), the separate top-k and
union kernels (17 and 64 tokens, and moe_route_topk + moe_union at any size),
the chunked union (4096 tokens: at least 4096 assignments), the router's
register GEMV (up to 16 tokens) and its tiled GEMM (above 16). Expert ids,
union, offsets, permutation and hit counters must equal the oracle's bit for
bit; gate weights agree to 2e-6 (exactly when every score is sigmoid(0)) and
layer outputs to the usual 2e-3 per token.
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

W_TOL = 2e-6
TOL = 2e-3
SIZES = [1, 2, 16, 17, 64, 4096]
KINDS = ["pairs", "zero", "steps"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tie_router(cfg, kind):
    """(Wr, b) float32 with exact ties of the given kind."""
    spec = cfg.layers[0]
    E, d = spec.n_experts, spec.d
    if kind == "pairs":
        wr, b = synth.router(cfg, 0)
        wr = wr.copy()
        b = np.zeros(E, np.float32) if b is None else b.copy()
        wr[1::2] = wr[0::2]
        b[1::2] = b[0::2]
        return wr, b
    wr = np.zeros((E, d), np.float32)
    if kind == "zero":
        return wr, np.zeros(E, np.float32)
    # steps: groups of four equal biases, the last group best; the groups'
    # scores must differ by far more than float32 rounding near 1
    return wr, (0.01 * (np.arange(E) // 4)).astype(np.float32)


def tie_tokens(cfg, kind, wr, b, N, k):
    """N tokens. For "pairs", tokens whose distinct scores (one per pair) have
    a gap below 1e-6 among the best ceil(k/2)+1 are redrawn from their next
    attempt (the redraw rule applied to the distinct values only); the other
    kinds give scores that do not depend on x."""
    c = dataclasses.replace(cfg, n_tokens=N)
    attempts = np.zeros(N, np.int64)
    x = synth.tokens(c, attempts)
    if kind != "pairs":
        return x
    kk = (k + 1) // 2
    flagged = lc.small_gap_tokens(oracle.router(x, wr, b)[:, 0::2], kk)
    while len(flagged):
        attempts[flagged] += 1
        assert attempts.max() < 64
        x[flagged] = synth.tokens(c, attempts)[flagged]
        flagged = flagged[lc.small_gap_tokens(oracle.router(x[flagged], wr, b)[:, 0::2], kk)]
    return x


def expected_routing(x, wr, b, k, E):
    s = oracle.router(x, wr, b)
    ids, w = oracle.topk(s, k)
    u, off, perm = oracle.union(ids, E)
    cnt = oracle.hit_count(ids, E)
    return s, dict(ids=ids, w=w, union_ids=u, offsets=off, perm=perm, counters=cnt)


def check_routing(got, ref, exact_w):
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    if exact_w:
        np.testing.assert_array_equal(got["w"], ref["w"])
    else:
        assert np.max(np.abs(got["w"].astype(np.float64) - ref["w"])) <= W_TOL
    np.testing.assert_array_equal(got["union_ids"], ref["union_ids"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["perm"], ref["perm"])
    np.testing.assert_array_equal(got["counters"], ref["counters"])


def route_only(x, wr, b, k, E, fused):
    """moe_route_union (fused) or moe_route_topk + moe_union + moe_hit_count."""
    dev = "cuda"
    N = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ids = torch.full((N, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((N, k), -7.0, dtype=torch.float32, device=dev)
    uid = torch.full((E,), -1, dtype=torch.int32, device=dev)
    nu = torch.full((1,), -1, dtype=torch.int32, device=dev)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((N * k,), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev)
    ws = torch.empty(moe.route_workspace_size(N, E), dtype=torch.uint8, device=dev)
    if fused:
        moe.route_union(xd, wrd, bd, k, ids, w, uid, nu, off, perm, cnt, ws)
    else:
        moe.route_topk(xd, wrd, bd, k, ids, w, ws)
        moe.union(ids, E, uid, nu, off, perm)
        moe.hit_count(ids, E, cnt)
    torch.cuda.synchronize()
    n = int(nu.item())
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), union_ids=uid.cpu().numpy()[:n],
                offsets=off.cpu().numpy(), perm=perm.cpu().numpy(),
                counters=cnt.cpu().numpy().astype(np.uint64))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N", SIZES)
def test_route_ties_decode_shapes(kind, N):
    """Routing alone on the decode layer's router (6144 x 256), k = 1, 2, 3, 8,
    through moe_route_union and through the three separate calls."""
    cfg = synth.CONFIGS["decode64"]
    E = cfg.layers[0].n_experts
    wr, b = tie_router(cfg, kind)
    for k in (1, 2, 3, 8):
        x = tie_tokens(cfg, kind, wr, b, N, k)
        s, ref = expected_routing(x, wr, b, k, E)
        if kind == "pairs" and k % 2 == 1:
            # the k-th pick is the lower id of a pair whose twin is left out
            last = ref["ids"][:, -1]
            assert np.all(last % 2 == 0)
            assert not np.any(ref["ids"] == (last + 1)[:, None])
        for fused in (True, False):
            got = route_only(x, wr, b, k, E, fused)
            check_routing(got, ref, exact_w=kind == "zero")
        say(f"[ties] {kind} N={N} k={k}: routing equals the oracle (fused and separate), "
            f"union {len(ref['union_ids'])}")


def _tiny_tie_layer(kind, N, k):
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=N, k=k)
    spec = cfg.layers[0]
    wr, b = tie_router(cfg, kind)
    x = tie_tokens(cfg, kind, wr, b, N, k)
    blocks, shared = lc.canonical_pool(cfg, 0)
    ref = oracle.layer_step(x, wr, b, k, blocks, shared, spec.d, spec.f, spec.wbits, spec.group)
    return cfg, spec, x, wr, b, blocks, shared, ref


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("k", [1, 2, 3])
def test_layer_ties_tiny(kind, N, k):
    """The whole layer on the tiny shapes (16 experts): the two-call step
    (moe_route_union + moe_expert_forward) and moe_layer_step, which at one
    or two tokens and k <= 2 takes the routing inside the gate/up launch."""
    cfg, spec, x, wr, b, blocks, shared, ref = _tiny_tie_layer(kind, N, k)
    pool = upload_pool(spec, blocks, shared)
    two = run_layer(pool, x, wr, b, k, fused_route=True)
    one = run_layer_step(pool, x, wr, b, k)
    for got in (two, one):
        check_routing(got, ref, exact_w=kind == "zero")
        err = lc.rel_err_rows(got["y"], ref["y"]).max()
        assert err <= TOL, f"max per-token relative error {err:.3e}"
    say(f"[ties] tiny {kind} N={N} k={k}: ids {ref['ids'][0].tolist()} ..., "
        f"union {ref['union_ids'].tolist()}, layer outputs within {TOL}")
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["pairs", "zero"])
@pytest.mark.parametrize("N,k", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_layer_step_ties_decode_shapes(kind, N, k):
    """moe_layer_step on the decode layer's shapes where the routing runs
    inside the gate/up GEMV launch. With the zero router both tokens of a
    two-token batch pick the same experts, so every routed item holds two
    tokens (the shared-expert path of the in-launch union)."""
    cfg = dataclasses.replace(synth.CONFIGS["decode1"], n_tokens=N, k=k)
    spec = cfg.layers[0]
    wr, b = tie_router(cfg, kind)
    x = tie_tokens(cfg, kind, wr, b, N, k)
    blocks, shared = lc.canonical_pool(cfg, 0)
    ref = oracle.layer_step(x, wr, b, k, blocks, shared, spec.d, spec.f, spec.wbits, spec.group)
    if kind == "zero":
        assert np.all(ref["ids"] == np.arange(k)[None, :])
    pool = upload_pool(spec, blocks, shared)
    one = run_layer_step(pool, x, wr, b, k)
    check_routing(one, ref, exact_w=kind == "zero")
    err = lc.rel_err_rows(one["y"], ref["y"]).max()
    assert err <= TOL, f"max per-token relative error {err:.3e}"
    two = run_layer(pool, x, wr, b, k, fused_route=True)
    for key in ("ids", "w", "union_ids", "offsets", "perm", "counters", "y"):
        np.testing.assert_array_equal(one[key], two[key], err_msg=key)
    say(f"[ties] decode shapes {kind} N={N} k={k}: ids {ref['ids'].tolist()}, "
        f"max rel err {err:.2e}")
    del pool
    torch.cuda.empty_cache()
