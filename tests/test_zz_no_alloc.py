"""moe_layer_step_noalloc (the layer step on the library's own workspace
array, for callers that cannot allocate) against moe_layer_step with a
caller-owned workspace, through the C ABI: two calls in a row on the GLM-5.2
decode shapes, the second with a smaller batch over the array the first one
left behind, each bit for bit equal to moe_layer_step (same kernels); a step
larger than the array is rejected with MOE_EWORKSPACE and writes nothing."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import int4_routed_expert_gemv_amd as moe
import oracle
import synth
from tests import layer_cases as lc
from tests.gpu_layer import run_layer_step, upload_pool

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc(pool, x, wr, b, k, counters):
    """moe_layer_step_noalloc on fresh output buffers (filled with values the
    call must overwrite)."""
    N, d = x.shape
    E = pool.desc.n_experts
    dev = "cuda"
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).to(dev)
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev)
    out = dict(ids=torch.full((N, k), -7, dtype=torch.int32, device=dev),
               w=torch.full((N, k), -7.0, dtype=torch.float32, device=dev),
               union_ids=torch.full((E,), -1, dtype=torch.int32, device=dev),
               n_union=torch.full((1,), -1, dtype=torch.int32, device=dev),
               offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
               perm=torch.full((N * k,), -1, dtype=torch.int32, device=dev),
               y=torch.full((N, d), float("nan"), dtype=torch.float32, device=dev))
    moe.layer_step_noalloc(pool.desc, xd, wrd, bd, k, out["ids"], out["w"], out["union_ids"],
                           out["n_union"], out["offsets"], out["perm"], counters, out["y"])
    torch.cuda.synchronize()
    nu = int(out["n_union"].item())
    got = {key: v.cpu().numpy() for key, v in out.items()}
    got["union_ids"] = got["union_ids"][:nu]
    got["n_union"] = nu
    got["counters"] = counters.cpu().numpy().astype(np.uint64)
    return got


def test_noalloc_equals_layer_step_two_calls():
    cfg = synth.CONFIGS["decode64"]          # 64 tokens, top-8: 22 MiB of workspace
    spec = cfg.layers[0]
    x, wr, b, _, _ = lc.layer_inputs(cfg, 0)
    blocks, shared = lc.canonical_pool(cfg, 0)
    small = dataclasses.replace(cfg, n_tokens=3)
    x2 = np.ascontiguousarray(x[5:8])        # a smaller batch for the second call
    ref2 = oracle.layer_step(x2, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits,
                             spec.group)
    pool = upload_pool(spec, blocks, shared)
    E = spec.n_experts
    for i, (xv, N) in enumerate(((x, cfg.n_tokens), (x2, small.n_tokens))):
        need = moe.layer_step_workspace_size(pool.desc, N, cfg.k)
        assert 0 < need <= moe.MOE_SCRATCH_BYTES
        say(f"[noalloc] call {i + 1}: {N} tokens, top-{cfg.k}, workspace {need} bytes")
        c_a = torch.zeros(E, dtype=torch.int64, device="cuda")
        c_b = torch.zeros(E, dtype=torch.int64, device="cuda")
        got = _noalloc(pool, xv, wr, b, cfg.k, c_a)
        want = run_layer_step(pool, xv, wr, b, cfg.k, counters=c_b)
        for key in ("ids", "w", "union_ids", "offsets", "perm", "counters", "y"):
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"call {i + 1}: {key}")
        assert got["n_union"] == want["n_union"]
        assert got["counters"].sum() == N * cfg.k
        say(f"[noalloc] call {i + 1} equals moe_layer_step bit for bit "
            f"(union {got['n_union']})")
    # the second, smaller call also against the oracle
    np.testing.assert_array_equal(got["ids"], ref2["ids"])
    np.testing.assert_array_equal(got["perm"], ref2["perm"])
    assert lc.rel_err_rows(got["y"], ref2["y"]).max() <= 2e-3
    del pool
    torch.cuda.empty_cache()


def test_noalloc_rejects_steps_larger_than_the_array():
    """256 tokens at top-8 on the GLM shapes need 88 MiB: MOE_EWORKSPACE,
    and the outputs keep what they held."""
    spec = synth.CONFIGS["decode64"].layers[0]
    desc = moe.PoolDesc(spec.d, spec.f, spec.n_experts, spec.wbits, spec.group, 1 << 20,
                        moe.block_bytes(spec.d, spec.f, spec.wbits, spec.group), None)
    N, k, E = 256, 8, spec.n_experts
    assert moe.layer_step_workspace_size(desc, N, k) > moe.MOE_SCRATCH_BYTES
    dev = "cuda"
    x = torch.zeros((N, spec.d), dtype=torch.float32, device=dev)
    wr = torch.zeros((E, spec.d), dtype=torch.float32, device=dev)
    ids = torch.full((N, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((N, k), -7.0, dtype=torch.float32, device=dev)
    uid = torch.full((E,), -1, dtype=torch.int32, device=dev)
    nu = torch.full((1,), -1, dtype=torch.int32, device=dev)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((N * k,), -1, dtype=torch.int32, device=dev)
    y = torch.full((N, spec.d), 3.0, dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_step_noalloc(desc, x, wr, None, k, ids, w, uid, nu, off, perm, None, y)
    assert e.value.status == moe.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()) and bool((ids == -7).all()) and int(nu.item()) == -1
