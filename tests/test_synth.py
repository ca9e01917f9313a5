"""The seeded input generator: SplitMix64 outputs and the drawn distributions."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLD, "splitmix64.json")))
    for i, v in enumerate(g["state0_outputs"]):
        assert synth.lib().synth_draw(0, i) == int(v, 16)


def test_counter_access_matches_sequence():
    k = synth.key(9, 1, 2, 3, 4)
    b = synth.random_bytes(k, 64)
    words = np.frombuffer(b.tobytes(), np.uint64)
    for i, w in enumerate(words):
        assert int(w) == synth.lib().synth_draw(k, i)


def test_distributions():
    k = synth.key(1, 0, 1, 0)
    x = synth.normal(k, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = synth.uniform(k, 200000, 0.002, 0.01)
    assert u.min() >= 0.002 and u.max() < 0.01 and abs(u.mean() - 0.006) < 1e-4
    b = synth.random_bytes(k, 1 << 16)
    nib = np.concatenate([b & 15, b >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * len(nib) / 16
    p = synth.permutation(k, 256)
    assert sorted(p.tolist()) == list(range(256))


def test_configs_and_zipf_bias():
    c = synth.CONFIGS["decode64"]
    wr, b = synth.router(c)
    assert wr.shape == (256, 6144) and abs(wr.std() - 0.05) < 1e-3
    rank = np.round(np.exp(-b / 1.1)).astype(int)
    assert sorted(rank.tolist()) == list(range(1, 257))
    wr4, b4 = synth.router(synth.CONFIGS["prefill4096"])
    assert np.all(b4 == 0)
    t = synth.CONFIGS["tiny"]
    pool = synth.expert_pool(t)
    assert pool.shape == (16, 61440)
    off = synth.canonical_offsets(t.layer)
    s = pool[0, off["gate_s"]:off["total"]].view(np.float32)
    assert s.min() >= 0.005 and s.max() < 0.02
    x1 = synth.tokens(t)
    x2 = synth.tokens(t, attempts=[0, 1, 0, 0])
    assert np.array_equal(x1[0], x2[0]) and not np.array_equal(x1[1], x2[1])
