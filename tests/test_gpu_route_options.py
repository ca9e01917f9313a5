"""GPU parity of the opt-in router variant (moe_route_topk_ex /
moe_route_union_ex: a bias that only steers the selection, weights
normalised over the chosen experts and scaled) against the CPU oracle
(oracle.topk_select), through the C ABI.

Expert ids, union, offsets, permutation and hit counters must match bit for
bit. The weights carry the scores' float32 error (at most 2e-6 absolute, the
bound the layer tests hold the raw scores to) through the normalisation:
w = scale * s_j / S with S the sum of the k chosen scores, so
|dw| <= scale * 2e-6 * (1 + k) / S, plus (k + 4) float32 roundings of w
(the sum, the division and the product). Tokens whose
oracle selection keys s + b have two of their top k+1 closer than 1e-6 are
left out of the id comparison (the same policy as the layer inputs), and the
rest must be most of the batch.
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
from tests.gpu_layer import upload_pool

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def clear_tokens(s, b, k, gap=1e-6):
    """Tokens whose top k+1 float32 keys s + b are at least `gap` apart."""
    key = np.sort((s + b[None, :]).astype(np.float32), axis=1)[:, ::-1][:, :k + 1]
    return np.all(np.diff(-key.astype(np.float64), axis=1) >= gap, axis=1)


def gpu_route(x, wr, b, k, options, fused=True):
    dev = "cuda"
    N = x.shape[0]
    E = wr.shape[0]
    xd, wrd, bd = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
                   for a in (x, wr, b))
    ws = torch.empty(max(1, moe.route_workspace_size(N, E)), dtype=torch.uint8, device=dev)
    ids = torch.full((N, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((N, k), -7.0, dtype=torch.float32, device=dev)
    uid = torch.full((E,), -7, dtype=torch.int32, device=dev)
    nu = torch.full((1,), -7, dtype=torch.int32, device=dev)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm = torch.full((N * k,), -7, dtype=torch.int32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev)
    if fused:
        moe.route_union(xd, wrd, bd, k, ids, w, uid, nu, off, perm, cnt, ws, options=options)
    else:
        moe.route_topk(xd, wrd, bd, k, ids, w, ws, options=options)
        moe.union(ids, E, uid, nu, off, perm)
        moe.hit_count(ids, E, cnt)
    torch.cuda.synchronize()
    n = int(nu.item())
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), union_ids=uid.cpu().numpy()[:n],
                offsets=off.cpu().numpy(), perm=perm.cpu().numpy(),
                counters=cnt.cpu().numpy().astype(np.uint64))


# decode-layer router (6144 x 256, Zipf log-popularity bias), batch sizes on
# every route path: the one-workgroup tail (up to 16 tokens), the separate
# top-k and union kernels, and the chunked union (from 4096 assignments)
@pytest.mark.parametrize("N,k,norm,scale", [(1, 1, False, 1.0), (1, 8, True, 2.5),
                                            (4, 8, True, 1.0), (16, 8, False, 2.5),
                                            (64, 8, True, 2.5), (600, 8, True, 2.5),
                                            (4096, 8, True, 2.5)])
@pytest.mark.parametrize("fused", [True, False])
def test_select_bias_route_against_oracle(N, k, norm, scale, fused):
    cfg = dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=N, k=k)
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    say(f"[route options] N={N} k={k} normalize={norm} scale={scale} fused={fused}")
    s = oracle.router(x, wr, None)
    ref_ids, ref_w = oracle.topk_select(s, b, k, normalize=norm, scale=scale)
    got = gpu_route(x, wr, b, k, dict(bias_select_only=1, normalize=int(norm), scale=scale),
                    fused=fused)
    ok = clear_tokens(s, b, k)
    assert ok.mean() >= 0.9, f"only {ok.mean():.3f} of the tokens have clear keys"
    np.testing.assert_array_equal(got["ids"][ok], ref_ids[ok])
    chosen = np.take_along_axis(s, ref_ids, axis=1).astype(np.float64)
    ssum = chosen.sum(axis=1, keepdims=True) if norm else np.ones((N, 1))
    tol = scale * 2e-6 * ((1 + k) if norm else 1) / ssum + (k + 4) * 2.0**-24 * np.abs(ref_w)
    dw = np.abs(got["w"].astype(np.float64) - ref_w)
    assert np.all(dw[ok] <= tol[ok]), f"weight error {np.max(dw[ok] / tol[ok]):.2f} x the bound"
    # the Union and Learn outputs are an integer function of the GPU's own ids
    uref, offref, permref = oracle.union(got["ids"], wr.shape[0])
    np.testing.assert_array_equal(got["union_ids"], uref)
    np.testing.assert_array_equal(got["offsets"], offref)
    np.testing.assert_array_equal(got["perm"], permref)
    np.testing.assert_array_equal(got["counters"], oracle.hit_count(got["ids"], wr.shape[0]))
    if norm:
        np.testing.assert_allclose(got["w"].astype(np.float64).sum(axis=1), scale, rtol=4e-6)
    say(f"[route options] ok ({ok.sum()} of {N} tokens compared)")


@pytest.mark.parametrize("N,k", [(1, 1), (8, 8), (600, 8)])
def test_default_options_equal_the_plain_calls(N, k):
    """moe_route_union_ex with the default options gives the plain call's
    outputs bit for bit."""
    cfg = dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=N, k=k)
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    a = gpu_route(x, wr, b, k, None)
    c = gpu_route(x, wr, b, k, dict(bias_select_only=0, normalize=0, scale=1.0))
    for key in a:
        np.testing.assert_array_equal(a[key], c[key])


def test_select_bias_layer_step_tiny():
    """The variant's routing feeding the expert step: the tiny layer with a
    seeded selection bias, against the oracle's layer on the oracle's ids."""
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=24, k=2)
    spec = cfg.layers[0]
    x, wr, _, _, _ = lc.layer_inputs(cfg, 0)
    b = (np.random.default_rng(5).standard_normal(spec.n_experts) * 0.5).astype(np.float32)
    s = oracle.router(x, wr, None)
    ref_ids, ref_w = oracle.topk_select(s, b, cfg.k, normalize=True, scale=2.5)
    ok = clear_tokens(s, b, cfg.k)
    assert ok.all()
    blocks, shared = lc.canonical_pool(cfg, 0)
    ref_y = oracle.expert_forward(blocks, shared, spec.d, spec.f, spec.wbits, spec.group, x,
                                  ref_ids, ref_w)
    pool = upload_pool(spec, blocks, shared)
    dev = "cuda"
    N, E, k = cfg.n_tokens, spec.n_experts, cfg.k
    xd, wrd, bd = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
                   for a in (x, wr, b))
    ws = torch.empty(max(moe.workspace_size(pool.desc, N, k), 1), dtype=torch.uint8, device=dev)
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    uid = torch.empty(E, dtype=torch.int32, device=dev)
    nu = torch.empty(1, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(N * k, dtype=torch.int32, device=dev)
    y = torch.empty((N, spec.d), dtype=torch.float32, device=dev)
    moe.route_union(xd, wrd, bd, k, ids, w, uid, nu, off, perm, None, ws,
                    options=dict(bias_select_only=1, normalize=1, scale=2.5))
    moe.expert_forward(pool.desc, xd, k, w, uid, nu, off, perm, y, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    err = lc.rel_err_rows(y.cpu().numpy(), ref_y)
    assert err.max() <= 2e-3, f"max per-token relative error {err.max():.3e}"


def clear_of_cut(s, b, k, p, rel=1e-5):
    """Tokens whose top-p decisions are not within `rel` of the threshold."""
    key = (s + (b[None, :] if b is not None else 0)).astype(np.float32)
    order = np.argsort(-key, axis=1, kind="stable")[:, :k]
    ranked = np.take_along_axis(s, order, axis=1).astype(np.float64)
    tot = ranked.sum(axis=1, keepdims=True)
    before = np.cumsum(ranked, axis=1) - ranked
    return np.all(np.abs(before[:, 1:] - p * tot) > rel * tot, axis=1)


@pytest.mark.parametrize("N", [1, 16, 64, 600, 4096])
@pytest.mark.parametrize("p,select", [(0.5, False), (0.9, True)])
def test_top_p_route_against_oracle(N, p, select):
    """The top-p cutoff: ids (-1 for dropped slots), weights (0 for them),
    union, permutation and counters that leave the dropped slots out."""
    k = 8
    cfg = dataclasses.replace(synth.CONFIGS["decode64"], n_tokens=N, k=k)
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    say(f"[top-p] N={N} p={p} select={select}")
    if select:
        s = oracle.router(x, wr, None)
        bsel = b
    else:
        s = oracle.router(x, wr, b)
        bsel = None
    ref_ids, ref_w = oracle.topk_select(s, bsel, k, top_p=p)
    got = gpu_route(x, wr, b, k, dict(bias_select_only=int(select), top_p=p))
    ok = clear_tokens(s, bsel if select else np.zeros(wr.shape[0], np.float32), k) & \
        clear_of_cut(s, bsel, k, p)
    assert ok.mean() >= 0.9, f"only {ok.mean():.3f} of the tokens are clear"
    np.testing.assert_array_equal(got["ids"][ok], ref_ids[ok])
    assert np.all(got["w"][got["ids"] < 0] == 0.0)
    kept = ok[:, None] & (ref_ids >= 0)
    dw = np.abs(got["w"].astype(np.float64) - ref_w)
    assert np.all(dw[kept] <= 2e-6 + 2.0**-23 * np.abs(ref_w[kept]))
    assert (got["ids"] < 0).any(), "the cutoff dropped nothing"
    uref, offref, permref = oracle.union(got["ids"], wr.shape[0])
    np.testing.assert_array_equal(got["union_ids"], uref)
    np.testing.assert_array_equal(got["offsets"], offref)
    np.testing.assert_array_equal(got["perm"][:offref[-1]], permref[:offref[-1]])
    np.testing.assert_array_equal(got["counters"], oracle.hit_count(got["ids"], wr.shape[0]))


@pytest.mark.parametrize("N,k,with_shared,p", [(1, 4, True, 0.6), (24, 4, True, 0.6),
                                               (1, 2, False, 0.5), (24, 3, False, 0.6)])
def test_top_p_layer_step_tiny(N, k, with_shared, p):
    """Dropped slots through the expert step (the combine kernel, and at one
    token without the shared expert the down kernel's direct combine; at
    k = 2 a cutoff of 0.5 always drops the second slot)."""
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=N, k=k)
    spec = cfg.layers[0]
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    s = oracle.router(x, wr, b)
    ref_ids, ref_w = oracle.topk_select(s, None, k, top_p=p)
    blocks, shared = lc.canonical_pool(cfg, 0)
    if not with_shared:
        shared = None
    ref_y = oracle.expert_forward(blocks, shared, spec.d, spec.f, spec.wbits, spec.group, x,
                                  ref_ids, ref_w)
    pool = upload_pool(spec, blocks, shared)
    dev = "cuda"
    E = spec.n_experts
    xd, wrd, bd = (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
                   for a in (x, wr, b))
    ws = torch.empty(max(moe.workspace_size(pool.desc, N, k), 1), dtype=torch.uint8, device=dev)
    ws.fill_(255)   # stale workspace: a dropped slot's expert row must never be read
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    uid = torch.empty(E, dtype=torch.int32, device=dev)
    nu = torch.empty(1, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(N * k, dtype=torch.int32, device=dev)
    y = torch.empty((N, spec.d), dtype=torch.float32, device=dev)
    moe.route_union(xd, wrd, bd, k, ids, w, uid, nu, off, perm, None, ws,
                    options=dict(top_p=p))
    moe.expert_forward(pool.desc, xd, k, w, uid, nu, off, perm, y, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    assert (ref_ids < 0).any()
    yv = y.cpu().numpy()
    assert np.all(np.isfinite(yv))
    err = lc.rel_err_rows(yv, ref_y)
    assert err.max() <= 2e-3, f"max per-token relative error {err.max():.3e}"
