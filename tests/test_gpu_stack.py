"""The 8-layer int4 stack + int8 draft layer workload (256 tokens, top-8,
Zipf(1.1) router bias per layer), teacher-forced: every GPU layer consumes the
oracle's normalised input of that layer, so each layer is compared on the same
input. Routing, union, permutation and the per-layer hit counters must match
bit for bit; each layer's output within 2e-3 (per token, normwise)."""
import json
import os
import sys
import time

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

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def progress(msg):
    """Progress on stdout and, when MOE_TEST_PROGRESS names a file, appended
    to it (a long run that captures stdout stays visibly alive)."""
    print(msg, flush=True)
    path = os.environ.get("MOE_TEST_PROGRESS")
    if path:
        with open(path, "a") as fh:
            fh.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


@pytest.mark.timeout(1200)
def test_stack8_draft_teacher_forced():
    cfg = synth.CONFIGS["stack8_draft"]
    gold = json.load(open(os.path.join(GOLD, "stack8_attempts.json")))
    assert gold["config"] == cfg.name
    attempts = np.array(gold["attempts"], np.int64)
    E = cfg.layer.n_experts
    counters = torch.zeros((len(cfg.layers), E), dtype=torch.int64, device="cuda")
    errs = []

    def on_layer(l, spec, a, ref, blocks, shared, wr, b):
        assert len(lc.small_gap_tokens(ref["scores"], cfg.k)) == 0
        pool = upload_pool(spec, blocks, shared)
        got = run_layer(pool, a, wr, b, cfg.k, counters=counters[l])
        check_routing(got, ref, E)
        errs.append(check_y(got["y"], ref["y"]))
        progress(f"[stack8] layer {l} (wbits {spec.wbits}): union {got['n_union']}, "
                 f"max rel err {errs[-1]:.2e}")
        del pool
        torch.cuda.empty_cache()

    progress("[stack8] start")
    flagged = lc.stack_chain(cfg, attempts, on_layer=on_layer)
    assert flagged == []
    c = counters.cpu().numpy()
    assert np.all(c.sum(axis=1) == cfg.n_tokens * cfg.k)


def test_residual_rmsnorm_matches_oracle():
    rng = np.random.default_rng(11)
    N, d = 37, 6144
    h = (3.0 * rng.standard_normal((N, d))).astype(np.float32)
    y = rng.standard_normal((N, d)).astype(np.float32)
    hd = torch.from_numpy(h).cuda()
    yd = torch.from_numpy(y).cuda()
    ad = torch.empty_like(hd)
    moe.residual_rmsnorm(hd, yd, ad, 1e-6)
    torch.cuda.synchronize()
    ref_h = h.astype(np.float64) + y.astype(np.float64)
    ref_a = oracle.rms_normalize(ref_h, 1e-6)
    np.testing.assert_allclose(hd.cpu().numpy(), ref_h, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(ad.cpu().numpy(), ref_a, rtol=2e-6, atol=2e-6)
    # without y: normalise only, h untouched
    h2 = torch.from_numpy(h).cuda()
    moe.residual_rmsnorm(h2, None, ad, 1e-6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h2.cpu().numpy(), h)
    np.testing.assert_allclose(ad.cpu().numpy(), oracle.rms_normalize(h.astype(np.float64), 1e-6),
                               rtol=2e-6, atol=2e-6)
