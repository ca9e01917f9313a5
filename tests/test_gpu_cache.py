"""Place stage on the GPU: an HBM cache of expert slots over pinned host
memory (moe_cache_*), with the expert math reading blocks through the slot
table. Placement must not change results: every layer step through the
cache equals, bit for bit, the same step with every expert resident, and
the oracle's layer step (routing bit for bit, outputs within 2e-3); the
hits, misses, copies and slot assignments follow the oracle's per-layer
LRU model (oracle.LruCache) call by call."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import int4_routed_expert_gemv_amd as moe
import oracle
import synth
from tests import layer_cases as lc
from tests.gpu_layer import upload_pool, workspace

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pinned_blocks(pool):
    """The pool's packed device-layout blocks copied back into pinned host memory."""
    host = torch.empty((pool.desc.n_experts, pool.stride), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool.pool.view(pool.desc.n_experts, pool.stride).cpu())
    return host


def step(desc, x, wr, b, k, ws, cache=None, counters=None, routing=None):
    """route_union -> (place) -> expert_forward on the current stream.
    routing: a dict that receives the routing outputs (host arrays)."""
    N, d = x.shape
    E = desc.n_experts
    dev = "cuda"
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    uid = torch.full((E,), -1, dtype=torch.int32, device=dev)
    nu = torch.zeros(1, dtype=torch.int32, device=dev)
    off = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    perm = torch.zeros(N * k, dtype=torch.int32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev) if counters is None else counters
    moe.route_union(x, wr, b, k, ids, w, uid, nu, off, perm, cnt, ws)
    missed = None
    union = None
    if cache is not None:
        n = int(nu.item())                      # the host needs the union to place it
        union = uid[:n].cpu().numpy()
        missed = cache.place(union, copy_stream=cache_stream(), compute_stream=None)
    y = torch.empty((N, d), dtype=torch.float32, device=dev)
    moe.expert_forward(desc, x, k, w, uid, nu, off, perm, y, ws)
    if routing is not None:
        torch.cuda.synchronize()
        n = int(nu.item())
        routing.update(ids=ids.cpu().numpy(), union_ids=uid.cpu().numpy()[:n],
                       offsets=off.cpu().numpy(), perm=perm.cpu().numpy())
    return y, union, missed


def check_against_oracle(x, wr, b, k, blocks, shared, spec, y, routing):
    """routing bit for bit and y within 2e-3 (per token) of the oracle's step"""
    ref = oracle.layer_step(x, wr, b, k, blocks, shared, spec.d, spec.f, spec.wbits, spec.group)
    for key in ("ids", "union_ids", "offsets", "perm"):
        np.testing.assert_array_equal(routing[key], ref[key], err_msg=key)
    err = lc.rel_err_rows(y, ref["y"]).max()
    assert err <= 2e-3, f"max per-token relative error {err:.3e}"
    return err


_copy_stream = None


def cache_stream():
    global _copy_stream
    if _copy_stream is None:
        _copy_stream = torch.cuda.Stream()   # default priority
    return _copy_stream


@pytest.mark.parametrize("N,k,slots", [(1, 1, 3), (4, 2, 8), (3, 4, 12), (64, 4, 16)])
def test_cache_steps_equal_resident_pool(N, k, slots):
    """Several batches through a cache of `slots` slots (tiny layer, 16
    experts; 64 tokens x 4 also runs the matrix-core passes through the slot
    table): outputs equal the resident pool's bit for bit, misses and hits
    follow the LRU model, and slot contents equal the experts' blocks."""
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=N * 6, k=k)
    spec = cfg.layers[0]
    x_all, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    blocks, shared = lc.canonical_pool(cfg, 0)
    blocks_c, shared_c = blocks.copy(), shared.copy()   # canonical copies for the oracle
    pool = upload_pool(spec, blocks, shared)
    host = pinned_blocks(pool)
    cache = moe.ExpertCache(pool.desc, slots, host)
    model = oracle.LruCache(slots, spec.n_experts)
    dev = "cuda"
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ws = workspace(pool, N, k)
    tot_h = tot_m = 0
    for it in range(6):
        x = torch.from_numpy(np.ascontiguousarray(x_all[it * N:(it + 1) * N])).to(dev)
        y_res, _, _ = step(pool.desc, x, wrd, bd, k, ws)
        rt = {}
        y_cache, union, missed = step(cache.desc, x, wrd, bd, k, ws, cache=cache, routing=rt)
        torch.cuda.synchronize()
        hits, misses = model.place([int(e) for e in union])
        tot_h += hits
        tot_m += misses
        err = check_against_oracle(x_all[it * N:(it + 1) * N], wr, b, k, blocks_c, shared_c,
                                   spec, y_cache.cpu().numpy(), rt)
        say(f"[cache] N={N} k={k} slots={slots} step {it}: union {len(union)} missed {missed} "
            f"(oracle model {misses}), max rel err {err:.2e}")
        assert missed == misses
        np.testing.assert_array_equal(cache.resident()[0], model.slot_of())
        np.testing.assert_array_equal(y_cache.cpu().numpy(), y_res.cpu().numpy())
    assert cache.stats() == (tot_h, tot_m)
    # every resident expert's slot holds its block
    table = cache.table.cpu().numpy()
    slots_host = cache.slots.view(slots, pool.stride).cpu()
    for e in range(spec.n_experts):
        if table[e] >= 0:
            assert torch.equal(slots_host[table[e]], host[e]), e
    cache.close()


def test_cache_rejects_union_larger_than_slots():
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=8, k=4)
    spec = cfg.layers[0]
    blocks, shared = lc.canonical_pool(cfg, 0)
    pool = upload_pool(spec, blocks, shared)
    cache = moe.ExpertCache(pool.desc, 2, pinned_blocks(pool))
    with pytest.raises(moe.MoeError) as e:
        cache.place(np.array([0, 1, 2], np.int32))
    assert e.value.status == moe.MOE_ESHAPE
    assert cache.stats() == (0, 0)
    assert cache.place(np.array([3, 3, 40, -1], np.int32)) == 1   # duplicates / out of range ignored
    cache.close()



def test_pinned_and_prefetched_experts():
    """Pins keep their slots through many unions; a prefetch followed by the
    Place of the same layer turns the predicted experts into hits (the Place
    waits for the prefetch's copies, so outputs still equal the resident
    pool's bit for bit); hit / miss counts follow the model; a union that
    needs more than the unpinned slots is rejected."""
    N, k, slots = 3, 2, 10   # a union (at most 6 experts) always fits the 7 unpinned slots
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=N * 10, k=k)
    spec = cfg.layers[0]
    x_all, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    blocks, shared = lc.canonical_pool(cfg, 0)
    blocks_c, shared_c = blocks.copy(), shared.copy()   # canonical copies for the oracle
    pool = upload_pool(spec, blocks, shared)
    host = pinned_blocks(pool)
    cache = moe.ExpertCache(pool.desc, slots, host)
    model = oracle.LruCache(slots, spec.n_experts)
    dev = "cuda"
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ws = workspace(pool, N, k)
    pins = np.array([5, 11, 2], np.int32)
    assert cache.pin(pins, copy_stream=cache_stream()) == model.pin([5, 11, 2]) == 3
    so0, pinned = cache.resident()
    assert sorted(np.nonzero(pinned)[0].tolist()) == [2, 5, 11]
    with pytest.raises(moe.MoeError) as e:   # 8 unpinned experts, 7 unpinned slots
        cache.place(np.array([0, 1, 3, 4, 6, 7, 8, 9, 5], np.int32))
    assert e.value.status == moe.MOE_ESHAPE
    tot_h = tot_m = 0
    rng = np.random.default_rng(4)
    for it in range(10):
        x = torch.from_numpy(np.ascontiguousarray(x_all[it * N:(it + 1) * N])).to(dev)
        if it % 2:
            # predict this batch's union with the batch itself (a perfect
            # lookahead) plus two random experts, and prefetch it
            ids_pred = torch.empty((N, k), dtype=torch.int32, device=dev)
            w_pred = torch.empty((N, k), dtype=torch.float32, device=dev)
            rws = torch.empty(moe.route_workspace_size(N, spec.n_experts), dtype=torch.uint8,
                              device=dev)
            moe.route_topk(x, wrd, bd, k, ids_pred, w_pred, rws)
            pred = [int(e) for e in dict.fromkeys(ids_pred.cpu().numpy().ravel().tolist())]
            pred += [int(e) for e in rng.integers(0, spec.n_experts, size=2)]
            n_pf = cache.prefetch(np.array(pred, np.int32), copy_stream=cache_stream())
            assert n_pf == model.prefetch(pred)
        y_res, _, _ = step(pool.desc, x, wrd, bd, k, ws)
        rt = {}
        y_cache, union, missed = step(cache.desc, x, wrd, bd, k, ws, cache=cache, routing=rt)
        torch.cuda.synchronize()
        hits, misses = model.place([int(e) for e in union])
        tot_h += hits
        tot_m += misses
        check_against_oracle(x_all[it * N:(it + 1) * N], wr, b, k, blocks_c, shared_c, spec,
                             y_cache.cpu().numpy(), rt)
        say(f"[pin/prefetch] step {it}: union {union.tolist()} missed {missed} "
            f"(oracle model {misses})")
        assert missed == misses
        np.testing.assert_array_equal(cache.resident()[0], model.slot_of())
        if it % 2:
            assert missed == 0   # every expert of the union was prefetched
        np.testing.assert_array_equal(y_cache.cpu().numpy(), y_res.cpu().numpy())
        so, pinned = cache.resident()
        assert all(so[e] == so0[e] and pinned[e] for e in (2, 5, 11))
    assert cache.stats() == (tot_h, tot_m)
    table = cache.table.cpu().numpy()
    so, _ = cache.resident()
    np.testing.assert_array_equal(table, so)
    slots_host = cache.slots.view(slots, pool.stride).cpu()
    for e in range(spec.n_experts):
        if table[e] >= 0:
            assert torch.equal(slots_host[table[e]], host[e]), e
    assert cache.pin(np.array([], np.int32)) == 0
    assert not cache.resident()[1].any()
    cache.close()


@pytest.mark.parametrize("N,k,slots,E", [(1, 1, 3, 16), (4, 2, 8, 16), (3, 4, 16, 16),
                                          (64, 4, 16, 16), (24, 3, 52, 64)])
def test_cache_forward_overlap(N, k, slots, E):
    """moe_cache_forward: the resident experts and the shared expert computed
    while the missing blocks are copied in, then the copied experts and the
    combine. Every step equals the resident pool bit for bit and the oracle's
    layer step; misses and slot assignments follow the oracle's LRU model
    (cold cache first, then partly warm; 16 slots over 16 experts ends fully
    resident, the no-copy path; 64 tokens, and 24 tokens over 64 experts with
    52 slots, run the matrix-core passes on partly cached unions).
    Odd steps prefetch part of the next union first, so the forward also
    meets prefetched blocks whose copies it must wait for."""
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=N * 8, k=k,
                              layers=(dataclasses.replace(base.layer, n_experts=E),))
    spec = cfg.layers[0]
    x_all, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    blocks, shared = lc.canonical_pool(cfg, 0)
    blocks_c, shared_c = blocks.copy(), shared.copy()
    pool = upload_pool(spec, blocks, shared)
    cache = moe.ExpertCache(pool.desc, slots, pinned_blocks(pool))
    model = oracle.LruCache(slots, spec.n_experts)
    dev = "cuda"
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ws = workspace(pool, N, k)
    tot_h = tot_m = 0
    for it in range(8):
        x = torch.from_numpy(np.ascontiguousarray(x_all[it * N:(it + 1) * N])).to(dev)
        y_res, _, _ = step(pool.desc, x, wrd, bd, k, ws)
        y_res = y_res.cpu().numpy()
        ids = torch.empty((N, k), dtype=torch.int32, device=dev)
        w = torch.empty((N, k), dtype=torch.float32, device=dev)
        uid = torch.full((E,), -1, dtype=torch.int32, device=dev)
        nu = torch.zeros(1, dtype=torch.int32, device=dev)
        off = torch.zeros(E + 1, dtype=torch.int32, device=dev)
        perm = torch.zeros(N * k, dtype=torch.int32, device=dev)
        moe.route_union(x, wrd, bd, k, ids, w, uid, nu, off, perm, None, ws)
        n = int(nu.item())
        union = uid[:n].cpu().numpy()
        if it % 2 == 1 and n > 1:
            pf = union[: n // 2]
            assert cache.prefetch(pf, copy_stream=cache_stream()) == model.prefetch(pf)
        y = torch.full((N, spec.d), float("nan"), dtype=torch.float32, device=dev)
        missed = cache.forward(x, k, w, uid, nu, off, perm, union, y, ws,
                               copy_stream=cache_stream())
        torch.cuda.synchronize()
        hits, misses = model.place([int(e) for e in union])
        tot_h += hits
        tot_m += misses
        rt = dict(ids=ids.cpu().numpy(), union_ids=union, offsets=off.cpu().numpy(),
                  perm=perm.cpu().numpy())
        err = check_against_oracle(x_all[it * N:(it + 1) * N], wr, b, k, blocks_c, shared_c,
                                   spec, y.cpu().numpy(), rt)
        say(f"[overlap] N={N} k={k} slots={slots} step {it}: union {n} missed {missed} "
            f"(oracle model {misses}), max rel err {err:.2e}")
        assert missed == misses
        np.testing.assert_array_equal(cache.resident()[0], model.slot_of())
        np.testing.assert_array_equal(y.cpu().numpy(), y_res)
    assert cache.stats() == (tot_h, tot_m)
    cache.close()


def test_cache_forward_argument_checks():
    """Refusals before anything changes: a union larger than the slots, a
    pool shape that does not match the cache's blocks, a missing workspace."""
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_tokens=4, k=2)
    spec = cfg.layers[0]
    blocks, shared = lc.canonical_pool(cfg, 0)
    pool = upload_pool(spec, blocks, shared)
    cache = moe.ExpertCache(pool.desc, 2, pinned_blocks(pool))
    dev = "cuda"
    E, N, k = spec.n_experts, 4, 2
    x = torch.zeros((N, spec.d), dtype=torch.float32, device=dev)
    w = torch.zeros((N, k), dtype=torch.float32, device=dev)
    uid = torch.zeros(E, dtype=torch.int32, device=dev)
    nu = torch.zeros(1, dtype=torch.int32, device=dev)
    off = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    perm = torch.zeros(N * k, dtype=torch.int32, device=dev)
    y = torch.zeros((N, spec.d), dtype=torch.float32, device=dev)
    ws = workspace(pool, N, k)
    with pytest.raises(moe.MoeError) as e:
        cache.forward(x, k, w, uid, nu, off, perm, np.array([0, 1, 2], np.int32), y, ws)
    assert e.value.status == moe.MOE_ESHAPE
    with pytest.raises(moe.MoeError) as e:
        cache.forward(x, k, w, uid, nu, off, perm, np.array([0], np.int32), y, ws[:16])
    assert e.value.status == moe.MOE_EWORKSPACE
    assert cache.stats() == (0, 0) and not (cache.resident()[0] >= 0).any()
    cache.close()
