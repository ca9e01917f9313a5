"""Runs one layer step on the GPU through the C ABI (binding in
int4_routed_expert_gemv_amd) and returns the results as numpy arrays."""
import numpy as np
import torch

import int4_routed_expert_gemv_amd as moe


def upload_pool(spec, blocks, shared, device="cuda"):
    return moe.DevicePool(spec.d, spec.f, spec.n_experts, spec.wbits, spec.group, blocks, shared,
                          device)


def workspace(pool, N, k, device="cuda"):
    n = max(moe.workspace_size(pool.desc, N, k), 1)
    return torch.empty(n, dtype=torch.uint8, device=device)


def run_layer(pool, x, wr, b, k, ids_in=None, w_in=None, counters=None, device="cuda",
              mfma_min_tokens=None, mfma_small_min_tokens=None, fused_route=False, ws=None):
    """route_topk (unless ids_in/w_in are given) -> union -> hit_count -> expert_forward
    (moe_expert_forward_ex with those thresholds when either is given; None
    leaves a threshold at its default). fused_route: route, union and count
    with one moe_route_union call instead. ws: a workspace to reuse."""
    N, d = x.shape
    E = pool.desc.n_experts
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
    if ws is None:
        ws = workspace(pool, N, k, device)
    union_ids = torch.full((E,), -1, dtype=torch.int32, device=device)
    n_union = torch.zeros(1, dtype=torch.int32, device=device)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=device)
    perm = torch.full((N * k,), -1, dtype=torch.int32, device=device)
    cnt = torch.zeros(E, dtype=torch.int64, device=device) if counters is None else counters
    if ids_in is None:
        wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(device)
        bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(device)
        ids = torch.empty((N, k), dtype=torch.int32, device=device)
        w = torch.empty((N, k), dtype=torch.float32, device=device)
        if fused_route:
            moe.route_union(xd, wrd, bd, k, ids, w, union_ids, n_union, offsets, perm, cnt, ws)
        else:
            moe.route_topk(xd, wrd, bd, k, ids, w, ws)
    else:
        assert not fused_route
        ids = torch.from_numpy(np.ascontiguousarray(ids_in, np.int32)).to(device)
        w = torch.from_numpy(np.ascontiguousarray(w_in, np.float32)).to(device)
    if not fused_route:
        moe.union(ids, E, union_ids, n_union, offsets, perm)
        moe.hit_count(ids, E, cnt)
    y = torch.empty((N, d), dtype=torch.float32, device=device)
    opts = None
    if mfma_min_tokens is not None or mfma_small_min_tokens is not None:
        opts = moe.ForwardOptions()
        opts.mfma_min_tokens = mfma_min_tokens or 0
        opts.mfma_small_min_tokens = mfma_small_min_tokens or 0
    moe.expert_forward(pool.desc, xd, k, w, union_ids, n_union, offsets, perm, y, ws,
                       options=opts)
    torch.cuda.synchronize()
    nu = int(n_union.item())
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), union_ids=union_ids.cpu().numpy()[:nu],
                n_union=nu, offsets=offsets.cpu().numpy(), perm=perm.cpu().numpy(),
                counters=cnt.cpu().numpy().astype(np.uint64), y=y.cpu().numpy(), counters_t=cnt)


def run_layer_step(pool, x, wr, b, k, counters=None, options=None, device="cuda"):
    """moe_layer_step on fresh output buffers (filled with values the call
    must overwrite); returns the results as numpy arrays."""
    N, d = x.shape
    E = pool.desc.n_experts
    dev = device
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    ids = torch.full((N, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((N, k), -7.0, dtype=torch.float32, device=dev)
    union_ids = torch.full((E,), -1, dtype=torch.int32, device=dev)
    n_union = torch.full((1,), -1, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((N * k,), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev) if counters is None else counters
    y = torch.full((N, d), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.layer_step_workspace_size(pool.desc, N, k), 1), dtype=torch.uint8,
                     device=dev)
    moe.layer_step(pool.desc, xd, wrd, bd, k, ids, w, union_ids, n_union, offsets, perm, cnt, y,
                   ws, options=options)
    torch.cuda.synchronize()
    nu = int(n_union.item())
    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), union_ids=union_ids.cpu().numpy()[:nu],
                n_union=nu, offsets=offsets.cpu().numpy(), perm=perm.cpu().numpy(),
                counters=cnt.cpu().numpy().astype(np.uint64), y=y.cpu().numpy(), counters_t=cnt)
