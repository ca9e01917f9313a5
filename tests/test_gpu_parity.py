"""GPU parity of the layer step against the CPU oracle, through the C ABI.

Integers (expert ids, union, offsets, permutation, hit counters) must match
bit for bit; float outputs must satisfy, for every token,
max_i |y - y_ref| / max_i |y_ref| <= 2e-3. The gate weights are the chosen
float32 scores and must agree to 2e-6 (they differ by float32 rounding
only). Inputs whose top-(k+1) scores are closer than 1e-6 are redrawn first
(tests/layer_cases.py).
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
from tests.gpu_layer import run_layer, upload_pool, workspace

pytestmark = pytest.mark.gpu

TOL = 2e-3
W_TOL = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_routing(got, ref, E):
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    assert np.max(np.abs(got["w"].astype(np.float64) - ref["w"])) <= W_TOL
    np.testing.assert_array_equal(got["union_ids"], ref["union_ids"])
    assert got["n_union"] == len(ref["union_ids"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["perm"], ref["perm"])
    np.testing.assert_array_equal(got["counters"], ref["counters"])


def check_y(y, ref_y, tol=TOL):
    err = lc.rel_err_rows(y, ref_y)
    assert np.all(np.isfinite(y))
    assert err.max() <= tol, f"max per-token relative error {err.max():.3e} > {tol}"
    return float(err.max())


def oracle_then_pool(cfg, layer=0, x=None):
    spec = cfg.layers[layer]
    if x is None:
        x, wr, b, _, nre = lc.layer_inputs(cfg, layer)
    else:
        wr, b = synth.router(cfg, layer)
        nre = 0
    blocks, shared = lc.canonical_pool(cfg, layer)
    return spec, x, wr, b, blocks, shared, nre


def full_parity(cfg, layer=0, mfma_min_tokens=None, mfma_small_min_tokens=None,
                fused_route=False):
    spec, x, wr, b, blocks, shared, nre = oracle_then_pool(cfg, layer)
    say(f"[{cfg.name}] N={cfg.n_tokens} k={cfg.k} d={spec.d} f={spec.f} E={spec.n_experts} "
        f"wbits={spec.wbits} G={spec.group} redrawn={nre}")
    ref = oracle.layer_step(x, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits,
                            spec.group)
    pool = upload_pool(spec, blocks, shared)   # packs the blocks in place: oracle first
    say(f"[{cfg.name}] oracle done, union={len(ref['union_ids'])}; running GPU step "
        f"(mfma_min_tokens={mfma_min_tokens}, mfma_small_min_tokens={mfma_small_min_tokens}, "
        f"fused_route={fused_route})")
    got = run_layer(pool, x, wr, b, cfg.k, mfma_min_tokens=mfma_min_tokens,
                    mfma_small_min_tokens=mfma_small_min_tokens, fused_route=fused_route)
    check_routing(got, ref, spec.n_experts)
    err = check_y(got["y"], ref["y"])
    say(f"[{cfg.name}] parity ok, max rel err {err:.2e}")
    return pool, x, wr, b, got, ref


def test_tiny_layer():
    full_parity(synth.CONFIGS["tiny"])


def test_decode1_layer():
    full_parity(synth.CONFIGS["decode1"])
    torch.cuda.empty_cache()


def test_decode64_layer():
    full_parity(synth.CONFIGS["decode64"])
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_prefill4096_layer():
    """Full-size prefill, every output compared: routing, union, permutation
    and counters over all 4096 tokens, and the layer output of all 4096
    tokens (every row of every 128-token item, every remainder item on the
    32-token pass, and the shared expert's 4096-token group). The oracle runs
    on chunks of 1024 tokens, which is exact because tokens do not interact."""
    cfg = synth.CONFIGS["prefill4096"]
    spec, x, wr, b, blocks, shared, nre = oracle_then_pool(cfg)
    say(f"[prefill4096] redrawn={nre}")
    s = oracle.router(x, wr, b)
    ids, w = oracle.topk(s, cfg.k)
    u, off, perm = oracle.union(ids, spec.n_experts)
    cnt = oracle.hit_count(ids, spec.n_experts)
    T = np.diff(off)
    say(f"[prefill4096] tokens per expert: min {T.min()} max {T.max()}; experts above 128 "
        f"tokens {int((T > 128).sum())}, with a remainder of at most 32 "
        f"{int(((T > 128) & (T % 128 > 0) & (T % 128 <= 32)).sum())}")
    y_ref = np.empty((cfg.n_tokens, spec.d), np.float64)
    for c0 in range(0, cfg.n_tokens, 1024):
        c1 = min(cfg.n_tokens, c0 + 1024)
        y_ref[c0:c1] = oracle.expert_forward(blocks, shared, spec.d, spec.f, spec.wbits,
                                             spec.group, x[c0:c1], ids[c0:c1], w[c0:c1])
        say(f"[prefill4096] oracle tokens {c0}..{c1 - 1} done")
    pool = upload_pool(spec, blocks, shared)
    say("[prefill4096] running GPU step")
    got = run_layer(pool, x, wr, b, cfg.k)
    ref = dict(ids=ids, w=w, union_ids=u, offsets=off, perm=perm, counters=cnt)
    check_routing(got, ref, spec.n_experts)
    err = check_y(got["y"], y_ref)
    say(f"[prefill4096] parity ok on all {cfg.n_tokens} tokens, max rel err {err:.2e}")
    del pool
    torch.cuda.empty_cache()


def test_draft_int8_layer():
    """The int8 per-row-scale draft layer at full shape with 64 tokens."""
    cfg = dataclasses.replace(synth.CONFIGS["stack8_draft"], n_tokens=64)
    full_parity(cfg, layer=8)
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ edge cases

def tiny(**kw):
    return dataclasses.replace(synth.CONFIGS["tiny"], **kw)


@pytest.mark.parametrize("N,k", [(1, 1), (5, 1), (6, 2), (33, 3), (64, 4), (100, 16)])
def test_tiny_ragged_batches(N, k):
    """Token counts that leave partial work items and partial router tiles,
    k from 1 to E (k = E routes every token to every expert)."""
    pool, *_ = full_parity(tiny(n_tokens=N, k=k))


# (128-token threshold, 32-token threshold): every expert on the 128-token
# matrix-core pass, every expert on the 32-token pass, every expert on the
# GEMV, and the three mixed by thresholds 3 and 2
PASSES = [(1, -1), (-1, 1), (-1, -1), (3, 2)]


@pytest.mark.parametrize("big,small", PASSES)
@pytest.mark.parametrize("N,k", [(7, 3), (64, 4), (200, 16)])
def test_tiny_forced_paths(N, k, big, small):
    """Each pass on its own agrees with the oracle; the batches give partly
    filled 32- and 128-token tiles and multi-tile experts."""
    full_parity(tiny(n_tokens=N, k=k), mfma_min_tokens=big, mfma_small_min_tokens=small)


@pytest.mark.parametrize("big,small", PASSES)
def test_decode64_forced_paths(big, small):
    full_parity(synth.CONFIGS["decode64"], mfma_min_tokens=big, mfma_small_min_tokens=small)
    torch.cuda.empty_cache()


def test_determinism_and_counter_accumulation():
    cfg = synth.CONFIGS["decode64"]
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    pool = upload_pool(spec, blocks, shared)
    r1 = run_layer(pool, x, wr, b, cfg.k)
    r2 = run_layer(pool, x, wr, b, cfg.k, counters=r1["counters_t"])
    for key in ("ids", "w", "union_ids", "offsets", "perm", "y"):
        np.testing.assert_array_equal(r1[key], r2[key])
    np.testing.assert_array_equal(r2["counters"], 2 * r1["counters"])
    assert r2["counters"].sum() == 2 * cfg.n_tokens * cfg.k
    del pool
    torch.cuda.empty_cache()


# one pass for every expert, so that the same kernels run whatever the
# token counts: GEMV only, 32-token MFMA only, 128-token MFMA only
SINGLE_PASS = [(-1, -1), (-1, 1), (1, -1)]


@pytest.mark.parametrize("big,small", SINGLE_PASS)
def test_zero_gate_equals_dropped_slot(big, small):
    """w[:, 1] = 0 with k = 2 gives bit for bit the k = 1 result on slot 0
    (within one pass: the passes round differently)."""
    cfg = tiny(n_tokens=12, k=2)
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    ids, w = oracle.topk(oracle.router(x, wr, b), 2)
    pool = upload_pool(spec, blocks, shared)
    w0 = w.copy()
    w0[:, 1] = 0.0
    r2 = run_layer(pool, x, wr, b, 2, ids_in=ids, w_in=w0, mfma_min_tokens=big,
                   mfma_small_min_tokens=small)
    r1 = run_layer(pool, x, wr, b, 1, ids_in=ids[:, :1].copy(), w_in=w[:, :1].copy(),
                   mfma_min_tokens=big, mfma_small_min_tokens=small)
    np.testing.assert_array_equal(r2["y"], r1["y"])


@pytest.mark.parametrize("big,small", SINGLE_PASS)
def test_batch_invariance(big, small):
    """A token's output does not depend on the other tokens of the batch
    (within one pass)."""
    cfg = synth.CONFIGS["decode64"]
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    pool = upload_pool(spec, blocks, shared)
    full = run_layer(pool, x, wr, b, cfg.k, mfma_min_tokens=big, mfma_small_min_tokens=small)
    sub = np.arange(40) + 7
    part = run_layer(pool, x[sub], wr, b, cfg.k, mfma_min_tokens=big,
                     mfma_small_min_tokens=small)
    np.testing.assert_array_equal(part["ids"], full["ids"][sub])
    np.testing.assert_array_equal(part["y"], full["y"][sub])
    del pool
    torch.cuda.empty_cache()


def test_zero_tokens_is_a_no_op():
    cfg = synth.CONFIGS["tiny"]
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    pool = upload_pool(spec, blocks, shared)
    r = run_layer(pool, x[:0], wr, b, 1)
    assert r["y"].shape == (0, spec.d) and r["counters"].sum() == 0


@pytest.mark.parametrize("big,small", [(None, None), (1, None), (2, 1), (7, 3), (33, 5),
                                       (-1, None), (None, -1), (-1, -1), (-1, 40)])
@pytest.mark.parametrize("N,k", [(40, 8), (100, 3), (129, 16)])
def test_workspace_size_covers_every_threshold(N, k, big, small):
    """The workspace is sized once per (pool, N, k) and must hold the work
    lists of every pair of thresholds a call can choose; run_layer allocates
    exactly moe_workspace_size bytes."""
    full_parity(tiny(n_tokens=N, k=min(k, 16)), mfma_min_tokens=big, mfma_small_min_tokens=small)


@pytest.mark.parametrize("group", [0, 32, 64, 128])
@pytest.mark.parametrize("big,small", PASSES)
def test_tiny_int8_passes(group, big, small):
    """int8 codes (the draft layer's format) on each pass alone and mixed,
    with per-row scales, groups finer than a 64-column unit (each code
    scaled) and groups of whole units (the 32-token pass's per-step scaling
    and bias chain)."""
    base = synth.CONFIGS["tiny"]
    spec = dataclasses.replace(base.layer, wbits=8, group=group, scale_lo=0.005 / 16,
                               scale_hi=0.02 / 16)
    cfg = dataclasses.replace(base, n_tokens=64, k=4, layers=(spec,))
    full_parity(cfg, mfma_min_tokens=big, mfma_small_min_tokens=small)


@pytest.mark.parametrize("wbits,group", [(4, 32), (8, 0)])
@pytest.mark.parametrize("k", [1, 3, 8])
def test_single_token_several_experts(wbits, group, k):
    """One token routed to k experts with d_ff of several units (the
    one-item-per-union-slot GEMV path), int4 and int8."""
    base = synth.CONFIGS["tiny"]
    spec = dataclasses.replace(base.layer, f=512, wbits=wbits, group=group,
                               scale_lo=base.layer.scale_lo / (16 if wbits == 8 else 1),
                               scale_hi=base.layer.scale_hi / (16 if wbits == 8 else 1))
    full_parity(dataclasses.replace(base, n_tokens=1, k=k, layers=(spec,)))


@pytest.mark.parametrize("N,k", [(1, 1), (4, 1), (3, 8), (16, 5), (17, 2), (64, 4), (600, 8),
                                 (1000, 16)])
def test_route_union_against_oracle(N, k):
    """moe_route_union (one call for route, union and counting; one tail
    workgroup up to 16 tokens, the separate kernels above, the chunked union
    from 4096 assignments) on the tiny layer."""
    full_parity(tiny(n_tokens=N, k=k), fused_route=True)


@pytest.mark.parametrize("N,k", [(1, 1), (1, 8), (8, 8), (16, 8), (17, 8), (512, 8), (601, 7),
                                 (4096, 8)])
@pytest.mark.parametrize("with_counters", [True, False])
def test_route_union_equals_separate_calls(N, k, with_counters):
    """Bit for bit the outputs of moe_route_topk, moe_union and moe_hit_count
    on the decode layer's router (6144 x 256), counters accumulated in place."""
    cfg = dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=N, k=k)
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    E = wr.shape[0]
    say(f"[route_union] N={N} k={k} counters={with_counters}")
    dev = "cuda"
    xd, wrd, bd = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev) for a in (x, wr, b))
    ws = torch.empty(max(1, moe.route_workspace_size(N, E)), dtype=torch.uint8, device=dev)
    outs = []
    for fused in (False, True):
        ids = torch.full((N, k), -7, dtype=torch.int32, device=dev)
        w = torch.full((N, k), -7.0, dtype=torch.float32, device=dev)
        uid = torch.full((E,), -7, dtype=torch.int32, device=dev)
        nu = torch.full((1,), -7, dtype=torch.int32, device=dev)
        off = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
        perm = torch.full((N * k,), -7, dtype=torch.int32, device=dev)
        cnt = torch.arange(E, dtype=torch.int64, device=dev) * 3 if with_counters else None
        if fused:
            moe.route_union(xd, wrd, bd, k, ids, w, uid, nu, off, perm, cnt, ws)
        else:
            moe.route_topk(xd, wrd, bd, k, ids, w, ws)
            moe.union(ids, E, uid, nu, off, perm)
            if with_counters:
                moe.hit_count(ids, E, cnt)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (ids, w, uid, nu, off, perm)] +
                    ([cnt.cpu().numpy()] if with_counters else []))
    for a, c in zip(*outs):
        np.testing.assert_array_equal(a, c)
    ref_ids, _ = oracle.topk(oracle.router(x, wr, b), k)
    np.testing.assert_array_equal(outs[1][0], ref_ids)


def test_workspace_reuse_across_sizes():
    """One workspace over calls of different sizes on the GEMV-only path:
    nothing a call leaves in the workspace changes the next call's result
    (each equals a call on a fresh workspace bit for bit)."""
    cfg = tiny(n_tokens=9, k=3)
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    pool = upload_pool(spec, blocks, shared)
    ws = workspace(pool, 9, 3)
    for n in (1, 9, 2, 9, 1):
        say(f"[reuse] N={n}")
        a = run_layer(pool, x[:n], wr, b, 3, mfma_min_tokens=-1, mfma_small_min_tokens=-1, ws=ws)
        c = run_layer(pool, x[:n], wr, b, 3, mfma_min_tokens=-1, mfma_small_min_tokens=-1)
        np.testing.assert_array_equal(a["y"], c["y"])


@pytest.mark.parametrize("N,k", [(1, 1), (1, 4), (3, 2)])
def test_without_shared_expert(N, k):
    """A pool with no shared expert: y is the gate-weighted sum of the routed
    experts alone."""
    cfg = tiny(n_tokens=N, k=k)
    spec, x, wr, b, blocks, _, _ = oracle_then_pool(cfg)
    say(f"[no shared] N={N} k={k}")
    ref = oracle.layer_step(x, wr, b, k, blocks, None, spec.d, spec.f, spec.wbits, spec.group)
    pool = upload_pool(spec, blocks, None)
    got = run_layer(pool, x, wr, b, k, fused_route=True)
    check_routing(got, ref, spec.n_experts)
    check_y(got["y"], ref["y"])


@pytest.mark.parametrize("wbits", [4, 8])
def test_single_token_zero_gate_equals_dropped_slot(wbits):
    """One token, k = 2 with the second gate weight zero: bit for bit the
    k = 1 result (that expert adds exact zeros in the combine)."""
    base = synth.CONFIGS["tiny"]
    spec = dataclasses.replace(base.layer, f=512, wbits=wbits, group=32 if wbits == 4 else 0,
                               scale_lo=base.layer.scale_lo / (16 if wbits == 8 else 1),
                               scale_hi=base.layer.scale_hi / (16 if wbits == 8 else 1))
    cfg = dataclasses.replace(base, n_tokens=1, k=2, layers=(spec,))
    _, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    ids, w = oracle.topk(oracle.router(x, wr, b), 2)
    pool = upload_pool(spec, blocks, shared)
    w0 = w.copy()
    w0[:, 1] = 0.0
    r2 = run_layer(pool, x, wr, b, 2, ids_in=ids, w_in=w0)
    r1 = run_layer(pool, x, wr, b, 1, ids_in=ids[:, :1].copy(), w_in=w[:, :1].copy())
    np.testing.assert_array_equal(r2["y"], r1["y"])


@pytest.mark.parametrize("E,N,k", [(1000, 2, 32), (1000, 3, 32), (1024, 1, 7), (65, 9, 7),
                                   (1000, 40, 32), (300, 4096, 8)])
def test_route_union_many_experts(E, N, k):
    """Expert counts that are not a multiple of 64, up to the largest
    supported, on both union paths of the route tail (one wave up to 64
    assignments, the workgroup above), the separate kernels (40 tokens), and
    the router's 64 x 64 tiles with a partly filled last expert tile (4096
    tokens, 300 experts)."""
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=N, k=k,
                              layers=(dataclasses.replace(base.layer, n_experts=E),))
    say(f"[many experts] E={E} N={N} k={k}")
    full_parity(cfg, fused_route=True)


@pytest.mark.parametrize("group", [64, 0, 256])
def test_group_sizes_every_pass(group):
    """Scale groups of 64 inputs (the container format the README's "Get
    started" names, gs64), one scale per row (0) and groups spanning two
    128-column unit steps (256), int4, on the decode layer's shapes: each
    pass alone and the default mix, against one oracle run. (Groups of 64
    scale each code on the matrix-core passes; 0 and 256 take the 32-token
    pass's per-step scaling and its bias chain.)"""
    base = synth.CONFIGS["decode64"]
    cfg = dataclasses.replace(base, layers=(dataclasses.replace(base.layers[0], group=group),))
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    say(f"[gs{group}] N={cfg.n_tokens} k={cfg.k} G={spec.group}")
    ref = oracle.layer_step(x, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits,
                            spec.group)
    pool = upload_pool(spec, blocks, shared)
    for big, small in [(-1, -1), (-1, 1), (1, -1), (None, None)]:
        got = run_layer(pool, x, wr, b, cfg.k, mfma_min_tokens=big, mfma_small_min_tokens=small)
        check_routing(got, ref, spec.n_experts)
        err = check_y(got["y"], ref["y"])
        say(f"[gs{group}] big={big} small={small} max rel err {err:.2e}")
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", [2, 3])
def test_small_verify_batches(N):
    """Two and three tokens of top-8 on the decode layer's shapes (a
    speculative verify batch): two tokens stay on the GEMV by default (items
    of two tokens), three take the 32-token pass for experts hit twice."""
    cfg = dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=N)
    full_parity(cfg)
    full_parity(cfg, fused_route=True)


def test_decode1_direct_combine_is_deterministic():
    """One token, top-1 with the shared expert: the down kernel adds the two
    gate-weighted rows into y with float atomics (two addends onto zero, the
    same sum in either order), so repeated runs give the same bits."""
    cfg = synth.CONFIGS["decode1"]
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    pool = upload_pool(spec, blocks, shared)
    first = run_layer(pool, x, wr, b, cfg.k, fused_route=True)
    for _ in range(5):
        again = run_layer(pool, x, wr, b, cfg.k, fused_route=True)
        np.testing.assert_array_equal(again["y"], first["y"])
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d,f,wbits,group", [(16384, 128, 4, 128), (128, 16384, 4, 128),
                                             (16384, 128, 8, 0), (128, 16384, 8, 0)])
def test_largest_model_dims(d, f, wbits, group):
    """d_model or d_ff at the largest size the library accepts (16384), int4
    with groups of 128 and int8 with per-row scales: the GEMV's staged
    activations and the matrix-core passes' hidden rows at their longest, on
    each pass alone and mixed, against one oracle run."""
    base = synth.CONFIGS["tiny"]
    div = 16 if wbits == 8 else 1
    spec = dataclasses.replace(base.layer, d=d, f=f, wbits=wbits, group=group,
                               scale_lo=0.005 / div, scale_hi=0.02 / div)
    cfg = dataclasses.replace(base, n_tokens=40, k=4, layers=(spec,))
    spec, x, wr, b, blocks, shared, _ = oracle_then_pool(cfg)
    say(f"[largest dims] d={d} f={f} wbits={wbits} G={group} N={cfg.n_tokens} k={cfg.k}")
    ref = oracle.layer_step(x, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits,
                            spec.group)
    pool = upload_pool(spec, blocks, shared)
    for big, small in PASSES + [(None, None)]:
        got = run_layer(pool, x, wr, b, cfg.k, mfma_min_tokens=big, mfma_small_min_tokens=small)
        check_routing(got, ref, spec.n_experts)
        err = check_y(got["y"], ref["y"])
        say(f"[largest dims] big={big} small={small} max rel err {err:.2e}")
    del pool
    torch.cuda.empty_cache()
