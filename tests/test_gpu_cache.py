"""Place stage on the GPU: an HBM cache of expert slots over pinned host
memory (moe_cache_*), with the expert math reading blocks through the slot
table. Placement must not change results: every layer step through the
cache equals, bit for bit, the same step with every expert resident; the
hit / miss accounting follows least-recently-used replacement (checked
against a plain model of it here)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import int4_routed_expert_gemv_amd as moe
import synth
from tests import layer_cases as lc
from tests.gpu_layer import upload_pool, workspace

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class LruModel:
    """Least-recently-used slots: hits are refreshed first; each miss takes
    the least recently used slot not held by the current union and not
    pinned (lowest slot index among equals). pin() places a set and keeps
    its slots; prefetch() places the longest prefix of its list that fits in
    the unpinned slots."""

    def __init__(self, n_slots):
        self.expert_in = [-1] * n_slots
        self.last = [0] * n_slots
        self.pinned = [False] * n_slots
        self.tick = 0

    def pin(self, ids):
        self.pinned = [False] * len(self.expert_in)
        _, misses = self.place(ids)
        for s, e in enumerate(self.expert_in):
            if e in set(ids):
                self.pinned[s] = True
        return misses

    def _unpinned_needed(self, ids):
        slot_of = {e: s for s, e in enumerate(self.expert_in) if e >= 0}
        return len({e for e in ids if not (e in slot_of and self.pinned[slot_of[e]])})

    def prefetch(self, ids):
        room = len(self.expert_in) - sum(self.pinned)
        take = 0
        for i in range(len(ids)):
            if self._unpinned_needed(ids[:i + 1]) > room:
                break
            take = i + 1
        return self.place(ids[:take])[1]

    def place(self, ids):
        self.tick += 1
        used = [False] * len(self.expert_in)
        slot_of = {e: s for s, e in enumerate(self.expert_in) if e >= 0}
        hits = misses = 0
        for e in ids:
            if e in slot_of and not used[slot_of[e]]:
                used[slot_of[e]] = True
                self.last[slot_of[e]] = self.tick
                hits += 1
        for e in ids:
            if e in slot_of:
                continue
            cands = [s for s in range(len(used)) if not used[s] and not self.pinned[s]]
            v = min(cands, key=lambda s: (self.last[s], s))
            if self.expert_in[v] >= 0:
                del slot_of[self.expert_in[v]]
            self.expert_in[v] = e
            slot_of[e] = v
            used[v] = True
            self.last[v] = self.tick
            misses += 1
        return hits, misses


def pinned_blocks(pool):
    """The pool's packed device-layout blocks copied back into pinned host memory."""
    host = torch.empty((pool.desc.n_experts, pool.stride), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool.pool.view(pool.desc.n_experts, pool.stride).cpu())
    return host


def step(desc, x, wr, b, k, ws, cache=None, counters=None):
    """route_union -> (place) -> expert_forward on the current stream."""
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
    return y, union, missed


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
    pool = upload_pool(spec, blocks, shared)
    host = pinned_blocks(pool)
    cache = moe.ExpertCache(pool.desc, slots, host)
    model = LruModel(slots)
    dev = "cuda"
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ws = workspace(pool, N, k)
    tot_h = tot_m = 0
    for it in range(6):
        x = torch.from_numpy(np.ascontiguousarray(x_all[it * N:(it + 1) * N])).to(dev)
        y_res, _, _ = step(pool.desc, x, wrd, bd, k, ws)
        y_cache, union, missed = step(cache.desc, x, wrd, bd, k, ws, cache=cache)
        torch.cuda.synchronize()
        hits, misses = model.place([int(e) for e in union])
        tot_h += hits
        tot_m += misses
        say(f"[cache] N={N} k={k} slots={slots} step {it}: union {len(union)} missed {missed} "
            f"(model {misses})")
        assert missed == misses
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
    pool = upload_pool(spec, blocks, shared)
    host = pinned_blocks(pool)
    cache = moe.ExpertCache(pool.desc, slots, host)
    model = LruModel(slots)
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
        y_cache, union, missed = step(cache.desc, x, wrd, bd, k, ws, cache=cache)
        torch.cuda.synchronize()
        hits, misses = model.place([int(e) for e in union])
        tot_h += hits
        tot_m += misses
        say(f"[pin/prefetch] step {it}: union {union.tolist()} missed {missed} (model {misses})")
        assert missed == misses
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
