"""The layer step (moe_route_union + moe_expert_forward, or moe_layer_step)
captured in a HIP graph and replayed.

Every entry point enqueues kernels on the caller's stream and nothing else (no
allocation, no memset, no host synchronisation), so a serving loop can capture
a step once and replay it. Each replay must give the same bits as the same
step run eagerly, with new token rows copied into the captured input between
replays, eager steps on other buffers and synchronisations in between, and the
hit counters must accumulate once per replay. The first replay is also held
against the oracle.
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


def _buffers(N, k, d, E):
    dev = "cuda"
    return dict(
        ids=torch.empty((N, k), dtype=torch.int32, device=dev),
        w=torch.empty((N, k), dtype=torch.float32, device=dev),
        union_ids=torch.full((E,), -1, dtype=torch.int32, device=dev),
        n_union=torch.zeros(1, dtype=torch.int32, device=dev),
        offsets=torch.zeros(E + 1, dtype=torch.int32, device=dev),
        perm=torch.full((N * k,), -1, dtype=torch.int32, device=dev),
        cnt=torch.zeros(E, dtype=torch.int64, device=dev),
        y=torch.empty((N, d), dtype=torch.float32, device=dev),
    )


def _step(pool, xd, wrd, bd, k, t, ws, opts, one_call=False):
    if one_call:
        moe.layer_step(pool.desc, xd, wrd, bd, k, t["ids"], t["w"], t["union_ids"], t["n_union"],
                       t["offsets"], t["perm"], t["cnt"], t["y"], ws, options=opts)
        return
    moe.route_union(xd, wrd, bd, k, t["ids"], t["w"], t["union_ids"], t["n_union"],
                    t["offsets"], t["perm"], t["cnt"], ws)
    moe.expert_forward(pool.desc, xd, k, t["w"], t["union_ids"], t["n_union"], t["offsets"],
                       t["perm"], t["y"], ws, options=opts)


def _ws(pool, N, k):
    # large enough for both forms of the step
    n = max(moe.workspace_size(pool.desc, N, k), moe.layer_step_workspace_size(pool.desc, N, k))
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def _snapshot(t):
    nu = int(t["n_union"].item())
    return dict(ids=t["ids"].cpu().numpy(), w=t["w"].cpu().numpy(),
                union_ids=t["union_ids"].cpu().numpy()[:nu], n_union=nu,
                offsets=t["offsets"].cpu().numpy(), perm=t["perm"].cpu().numpy(),
                y=t["y"].cpu().numpy(), cnt=t["cnt"].cpu().numpy())


def _same(a, b):
    for key in ("ids", "w", "union_ids", "offsets", "perm", "y"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert a["n_union"] == b["n_union"]


def _case(name, n_tokens=None, k=None):
    """The workload's config, with n_tokens and top-k replaced when given."""
    cfg = synth.CONFIGS[name]
    if n_tokens is not None:
        cfg = dataclasses.replace(cfg, n_tokens=n_tokens, k=k)
    return cfg


# one token top-1 (GEMV, direct combine), 64 tokens top-8 (the 32-token
# pass), 300 tokens top-4 over 16 experts with every expert on the 128-token
# pass, and 20 tokens top-8 (the router's workgroup-tiled path and the
# separate union kernel) with the default passes
CASES = [("decode1", None, None, None, False, False), ("decode64", None, None, None, False, False),
         ("tiny", 300, 4, 1, False, False), ("tiny", 20, 8, None, False, False),
         # moe_layer_step: one and two tokens (routing inside the gate/up
         # launch), 20 tokens
         ("decode1", None, None, None, True, False), ("tiny", 1, 4, None, True, False),
         ("tiny", 2, 8, None, True, False), ("tiny", 20, 8, None, True, False),
         # two identical tokens: routed items of two tokens inside the launch
         ("tiny", 2, 1, None, True, True), ("tiny", 2, 2, None, True, True),
         ("decode64", 2, 2, None, True, True)]


@pytest.mark.parametrize("name,n_tokens,k,big,one_call,dup", CASES)
def test_graph_replay_equals_eager(name, n_tokens, k, big, one_call, dup):
    cfg = _case(name, n_tokens, k)
    opts = None
    if big is not None:
        opts = moe.ForwardOptions()
        opts.mfma_min_tokens = big
        opts.mfma_small_min_tokens = -1
    spec = cfg.layers[0]
    N, k, d, E = cfg.n_tokens, cfg.k, spec.d, spec.n_experts
    say(f"[graph] {name} N={N} k={k} d={d} f={spec.f} E={E} mfma_min_tokens={big} "
        f"one_call={one_call} dup={dup}")
    x0, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    if dup:  # every token a copy of token 0: the tokens share their experts
        x0 = np.ascontiguousarray(np.broadcast_to(x0[:1], x0.shape))
    blocks, shared = lc.canonical_pool(cfg, 0)
    ref = oracle.layer_step(x0, wr, b, k, blocks, shared, spec.d, spec.f, spec.wbits, spec.group)
    pool = upload_pool(spec, blocks, shared)
    x1 = np.ascontiguousarray(-x0[::-1])           # a second batch: other experts
    xs = [torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda() for v in (x0, x1)]
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).cuda()
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b, np.float32)).cuda()

    # eager results of both batches, each on fresh counters
    eager = []
    for xv in xs:
        t = _buffers(N, k, d, E)
        _step(pool, xv, wrd, bd, k, t, _ws(pool, N, k), opts, one_call)
        torch.cuda.synchronize()
        eager.append(_snapshot(t))

    # capture one step on static buffers
    st = _buffers(N, k, d, E)
    ws = _ws(pool, N, k)
    xd = xs[0].clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(pool, xd, wrd, bd, k, st, ws, opts, one_call)
    torch.cuda.synchronize()
    st["cnt"].zero_()

    order = [0, 1, 0, 1, 1]
    other = _buffers(N, k, d, E)
    other_ws = _ws(pool, N, k)
    for r, i in enumerate(order):
        xd.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(st)
        _same(got, eager[i])
        if r == 0:
            np.testing.assert_array_equal(got["ids"], ref["ids"])
            np.testing.assert_array_equal(got["perm"], ref["perm"])
            err = lc.rel_err_rows(got["y"], ref["y"]).max()
            assert err <= 2e-3, f"max per-token relative error {err:.3e}"
        # eager work of the program between replays, on other buffers
        _step(pool, xs[1 - i], wrd, bd, k, other, other_ws, opts, one_call)
        torch.cuda.synchronize()
        _same(_snapshot(other), eager[1 - i])
        say(f"[graph] {name} replay {r} (batch {i}) equals the eager step")
    want = sum(eager[i]["cnt"] for i in order)
    np.testing.assert_array_equal(st["cnt"].cpu().numpy(), want)
    del g, pool
    torch.cuda.empty_cache()
