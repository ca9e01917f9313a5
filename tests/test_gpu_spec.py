"""Layer stacks and the speculative-decoding flow, through moe_stack_forward.

The Colibri README ("Speculative decoding, honestly") drafts tokens with the
int8 MTP head and verifies them as one batch on the main layers with the same
kernels. Without trained weights there are no tokens to accept or reject, so
the flow here is the arithmetic of it on synthetic layers:
  draft:  g_0 = h, g_i = g_(i-1) + draft(rms(g_(i-1))) for i = 1 .. D, one
          token at a time through the int8 draft-head layer;
  verify: the batch [g_0, g_1, .., g_D] (1 + D tokens) through the 8 int4
          layers of the stack, chained by the residual RMS norm.

Parity is teacher-forced, as for the stack workload: every GPU layer step
consumes the oracle's normalised input of that step (routing bit for bit,
outputs within 2e-3 per token). The start token is redrawn until every draft
step keeps its top-k gaps; a verify token whose best scores fall within 1e-6
at some layer (the verify tokens follow from the drafts and cannot be redrawn
one by one) is left out of that layer's comparison, as the redraw rule leaves
such tokens out of the parity contract. The free-running GPU flow (moe_stack_forward
for each draft step and for the verify batch) must equal the same steps made
one call at a time (moe_residual_rmsnorm + moe_layer_step) bit for bit.
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
from tests.gpu_layer import run_layer, upload_pool
from tests.test_gpu_parity import check_routing, check_y

pytestmark = pytest.mark.gpu

EPS = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_layer(cfg, l, spec, blocks, shared, wr, b):
    pool = upload_pool(spec, blocks, shared)
    wrd = torch.from_numpy(np.ascontiguousarray(wr, np.float32)).cuda()
    bd = torch.from_numpy(np.ascontiguousarray(b, np.float32)).cuda()
    cnt = torch.zeros(spec.n_experts, dtype=torch.int64, device="cuda")
    return dict(pool=pool, wr=wrd, b=bd, cnt=cnt)


def stack_call(dls, h, k):
    """moe_stack_forward of h (a device tensor, updated) through the layers dls."""
    layers = moe.layer_descs([(d["pool"].desc, d["wr"], d["b"], d["cnt"]) for d in dls])
    ws = torch.empty(moe.stack_workspace_size(layers, h.shape[0], k), dtype=torch.uint8,
                     device="cuda")
    ids = torch.empty((len(dls), h.shape[0], k), dtype=torch.int32, device="cuda")
    moe.stack_forward(layers, h, k, ws, topk_ids_out=ids, eps=EPS)
    return ids


def one_call_at_a_time(dls, h, k):
    """the same chain through moe_residual_rmsnorm and moe_layer_step, one
    call each"""
    N, d = h.shape
    E = dls[0]["pool"].desc.n_experts
    a = torch.empty_like(h)
    y = torch.empty_like(h)
    out_ids = []
    for l, dl in enumerate(dls):
        moe.residual_rmsnorm(h, y if l else None, a, EPS)
        ids = torch.empty((N, k), dtype=torch.int32, device="cuda")
        w = torch.empty((N, k), dtype=torch.float32, device="cuda")
        uid = torch.empty(E, dtype=torch.int32, device="cuda")
        nu = torch.empty(1, dtype=torch.int32, device="cuda")
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(N * k, dtype=torch.int32, device="cuda")
        ws = torch.empty(moe.layer_step_workspace_size(dl["pool"].desc, N, k), dtype=torch.uint8,
                         device="cuda")
        moe.layer_step(dl["pool"].desc, a, dl["wr"], dl["b"], k, ids, w, uid, nu, off, perm,
                       dl["cnt"], y, ws)
        out_ids.append(ids)
    moe.residual_rmsnorm(h, y, a, EPS)
    return torch.stack(out_ids)


@pytest.mark.parametrize("N,k", [(1, 1), (2, 2), (8, 3), (40, 4)])
def test_stack_forward_equals_layer_calls_and_oracle(N, k):
    """Three tiny layers chained by moe_stack_forward: bit for bit the chain
    of single calls (outputs, ids, counters); each layer teacher-forced
    against the oracle chain."""
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, n_tokens=N, k=k, layers=(base.layer,) * 3)
    attempts = np.zeros(N, np.int64)
    x = synth.tokens(cfg, attempts)
    dls, dls2 = [], []
    flagged = []

    def on_layer(l, spec, a, ref, blocks, shared, wr, b):
        flagged.extend(lc.small_gap_tokens(ref["scores"], k).tolist())
        dl = device_layer(cfg, l, spec, blocks, shared, wr, b)
        got = run_layer(dl["pool"], a, wr, b, k)        # teacher-forced: the oracle's a_l
        if not flagged:
            check_routing(got, ref, spec.n_experts)
            check_y(got["y"], ref["y"])
        dls.append(dl)
        dls2.append(dict(dl, cnt=torch.zeros_like(dl["cnt"])))

    lc.stack_chain(cfg, attempts, on_layer=on_layer)
    h1 = torch.from_numpy(x).cuda()
    h2 = h1.clone()
    ids1 = stack_call(dls, h1, k)
    ids2 = one_call_at_a_time(dls2, h2, k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h1.cpu().numpy(), h2.cpu().numpy())
    np.testing.assert_array_equal(ids1.cpu().numpy(), ids2.cpu().numpy())
    for a_, b_ in zip(dls, dls2):
        np.testing.assert_array_equal(a_["cnt"].cpu().numpy(), b_["cnt"].cpu().numpy())
    say(f"[stack] N={N} k={k}: moe_stack_forward equals the single calls; redrawn gaps "
        f"{len(flagged)} (teacher-forced parity skipped for those layers)")


@pytest.fixture(scope="module")
def spec_flow():
    """The stack workload's pools on the GPU and the oracle's draft and
    verify flows for D = 1 and D = 4 drafts, with each GPU step checked
    teacher-forced as its layer is built."""
    cfg = synth.CONFIGS["stack8_draft"]
    k = cfg.k
    L = len(cfg.layers)
    draft_l = L - 1                     # the int8 draft-head layer
    # a start token whose draft and verify steps all keep their top-k gaps
    # (redrawn otherwise): one token, drafted for up to 4 steps
    c1 = dataclasses.replace(cfg, n_tokens=1)
    attempt = 0
    wr_d, b_d = synth.router(cfg, draft_l)
    sd = cfg.layers[draft_l]
    blocks_d, shared_d = lc.canonical_pool(cfg, draft_l)
    while True:
        h0 = synth.tokens(c1, np.array([attempt], np.int64)).astype(np.float64)
        g = [h0]
        refs_d, ok = [], True
        for i in range(4):
            a = oracle.rms_normalize(g[-1], EPS)
            ref = oracle.layer_step(a, wr_d, b_d, k, blocks_d, shared_d, sd.d, sd.f, sd.wbits,
                                    sd.group)
            ok &= len(lc.small_gap_tokens(ref["scores"], k)) == 0
            refs_d.append((a, ref))
            g.append(g[-1] + ref["y"])
        if ok:
            break
        attempt += 1
        assert attempt < 32
    say(f"[spec] start token attempt {attempt}; drafting through the int8 layer")
    dl_draft = device_layer(cfg, draft_l, sd, blocks_d, shared_d, wr_d, b_d)
    del blocks_d
    # draft steps on the GPU, teacher-forced
    for i, (a, ref) in enumerate(refs_d):
        got = run_layer(dl_draft["pool"], a, wr_d, b_d, k)
        check_routing(got, ref, sd.n_experts)
        err = check_y(got["y"], ref["y"])
        say(f"[spec] draft step {i + 1}: ids {ref['ids'][0].tolist()}, max rel err {err:.2e}")
    # verify batches: [g_0 .. g_D] for D = 1 and 4, through the int4 layers
    hs = {D: np.concatenate(g[:D + 1], axis=0) for D in (1, 4)}
    gaps = {D: 0 for D in hs}
    dls = []
    for l in range(draft_l):
        spec = cfg.layers[l]
        wr, b = synth.router(cfg, l)
        blocks, shared = lc.canonical_pool(cfg, l)
        refs = {}
        for D, h in hs.items():
            a = oracle.rms_normalize(h, EPS)
            refs[D] = (a, oracle.layer_step(a, wr, b, k, blocks, shared, spec.d, spec.f,
                                            spec.wbits, spec.group))
        dl = device_layer(cfg, l, spec, blocks, shared, wr, b)
        del blocks
        for D, (a, ref) in refs.items():
            bad = lc.small_gap_tokens(ref["scores"], k)
            gaps[D] += len(bad)
            got = run_layer(dl["pool"], a, wr, b, k)
            keep = np.setdiff1d(np.arange(D + 1), bad)
            # tokens with a gap below 1e-6 at this layer may rank either way
            np.testing.assert_array_equal(got["ids"][keep], ref["ids"][keep])
            if len(bad) == 0:
                check_routing(got, ref, spec.n_experts)
            check_y(got["y"][keep], ref["y"][keep])
            hs[D] = hs[D] + ref["y"]
        say(f"[spec] verify layer {l}: teacher-forced parity ok for 2 and 5 tokens")
        dls.append(dl)
        torch.cuda.empty_cache()
    return dict(cfg=cfg, k=k, dl_draft=dl_draft, dls=dls, h0=h0.astype(np.float32), gaps=gaps)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("D", [1, 4])
def test_draft_verify_flow(spec_flow, D):
    """The free-running GPU flow (D draft steps, then the verify batch)
    through moe_stack_forward equals the same steps made one call at a
    time, bit for bit; the teacher-forced parity ran in the fixture."""
    k = spec_flow["k"]
    dd = spec_flow["dl_draft"]
    g1 = [torch.from_numpy(spec_flow["h0"]).cuda()]
    g2 = [g1[0].clone()]
    for i in range(D):
        n1, n2 = g1[-1].clone(), g2[-1].clone()
        stack_call([dd], n1, k)
        one_call_at_a_time([dict(dd, cnt=torch.zeros_like(dd["cnt"]))], n2, k)
        g1.append(n1)
        g2.append(n2)
    v1 = torch.cat(g1, 0).contiguous()
    v2 = torch.cat(g2, 0).contiguous()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(v1.cpu().numpy(), v2.cpu().numpy())
    dls = spec_flow["dls"]
    ids1 = stack_call(dls, v1, k)
    ids2 = one_call_at_a_time([dict(d, cnt=torch.zeros_like(d["cnt"])) for d in dls], v2, k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(v1.cpu().numpy(), v2.cpu().numpy())
    np.testing.assert_array_equal(ids1.cpu().numpy(), ids2.cpu().numpy())
    assert np.all(np.isfinite(v1.cpu().numpy()))
    say(f"[spec] D={D}: verify batch of {D + 1} tokens through {len(dls)} layers, stack call "
        f"equals the single calls")
