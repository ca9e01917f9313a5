"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle with a closed form, a brute-force
enumeration, exact integer arithmetic, a special case that reduces to a
library routine, or an invariant of the layer. They are chosen so that a
dropped term, a wrong sign, index or orientation, or a swapped operand
fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from tests.canon import make_block, pack_codes, scales_shape

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LN3 = math.log(3.0)


# ---------------------------------------------------------------- router

def test_router_special_values():
    """sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4, 1/4; saturation at +-20."""
    E, d = 5, 8
    wr = np.zeros((E, d), np.float32)
    b = np.array([0.0, LN3, -LN3, 20.0, -20.0], np.float32)
    s = oracle.router(np.zeros((1, d), np.float32), wr, b)
    assert s[0, 0] == np.float32(0.5)
    assert s[0, 1] == np.float32(0.75)
    assert s[0, 2] == np.float32(0.25)
    assert s[0, 3] == np.float32(1.0)          # 1 - 2e-9 rounds to 1 in float32
    assert abs(float(s[0, 4]) - 2.0611536e-09) < 1e-15
    # no bias behaves as a zero bias
    s0 = oracle.router(np.zeros((1, d), np.float32), wr, None)
    assert np.all(s0 == np.float32(0.5))


def test_router_orientation():
    """l[t][e] = b[e] + sum_i Wr[e][i] x[t][i]: a one-hot token picks a column of Wr,
    and the row index of Wr is the expert."""
    E, d = 6, 9
    wr = np.zeros((E, d), np.float32)
    wr[2, 5] = LN3 / 2
    x = np.zeros((3, d), np.float32)
    x[0, 5] = 2.0     # token 0 hits Wr[2][5]
    x[1, 2] = 2.0     # token 1 would hit Wr[5][2] if the matrix were transposed
    s = oracle.router(x, wr, np.zeros(E, np.float32))
    expect = np.full((3, E), 0.5, np.float32)
    expect[0, 2] = 0.75
    np.testing.assert_array_equal(s, expect)


def test_router_matches_exact_sum_and_expit():
    """Against a correctly rounded sum of the exact float32 products (math.fsum)
    and scipy's expit: equal to within one float32 ulp."""
    rng = np.random.default_rng(1)
    N, E, d = 5, 7, 300
    x = rng.standard_normal((N, d)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((E, d))).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    s, logits = oracle.router(x, wr, b, return_logits=True)
    for t in range(N):
        for e in range(E):
            l = math.fsum([float(b[e])] + [float(wr[e, i]) * float(x[t, i]) for i in range(d)])
            assert abs(logits[t, e] - l) <= 1e-12 * (1 + abs(l))
            ref = np.float32(expit(l))
            assert abs(int(s[t, e].view(np.int32)) - int(ref.view(np.int32))) <= 1


# ---------------------------------------------------------------- top-k

def _brute_topk(srow, k):
    """The unique k-subset whose members all outrank every non-member under
    (score desc, id asc), listed in rank order."""
    E = len(srow)
    key = lambda e: (-float(srow[e]), e)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(key(a) < key(b) for a in S for b in rest):
            found.append(sorted(S, key=key))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("k", [1, 2, 3])
def test_topk_brute_force_with_ties(k):
    rng = np.random.default_rng(10 + k)
    E, N = 16, 40
    # few distinct levels -> many exact ties
    s = rng.integers(0, 5, size=(N, E)).astype(np.float32) / np.float32(4.0)
    ids, w = oracle.topk(s, k)
    for t in range(N):
        best = _brute_topk(s[t], k)
        assert list(ids[t]) == best
        np.testing.assert_array_equal(w[t], s[t, best])


def test_topk_all_equal_takes_lowest_ids():
    s = np.full((2, 16), 0.5, np.float32)
    ids, w = oracle.topk(s, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == 0.5)


# ---------------------------------------------------------------- router variant: selection-only bias

def test_topk_select_hand_computed():
    """The opt-in variant on a four-expert example worked by hand
    (tests/golden/route_select_hand.json)."""
    with open(os.path.join(GOLD, "route_select_hand.json")) as fh:
        g = json.load(fh)
    s = np.array([g["scores"]], np.float32)
    b = np.array(g["bias"], np.float32)
    ids, w = oracle.topk_select(s, b, g["k"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_array_equal(w[0], np.array(g["w_raw"], np.float32))
    ids, w = oracle.topk_select(s, b, g["k"], scale=g["scale"])
    np.testing.assert_allclose(w[0], g["w_scaled"], rtol=1e-7)
    ids, w = oracle.topk_select(s, b, g["k"], normalize=True, scale=g["scale"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], g["w_normalized"], rtol=1e-6)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_topk_select_brute_force_with_ties(k):
    """The chosen set is the unique k-subset whose float32 keys s + b all
    outrank the rest (ties to the lower id); the weights are the unbiased
    scores of the chosen experts."""
    rng = np.random.default_rng(50 + k)
    E, N = 12, 40
    s = (rng.integers(1, 6, size=(N, E)).astype(np.float32) / np.float32(8.0))
    b = (rng.integers(-2, 3, size=E).astype(np.float32) / np.float32(8.0))
    ids, w = oracle.topk_select(s, b, k)
    for t in range(N):
        key = (s[t] + b).astype(np.float32)   # numpy float32 addition
        best = _brute_topk(key, k)
        assert list(ids[t]) == best
        np.testing.assert_array_equal(w[t], s[t, best])


def test_topk_select_reduces_to_default_without_bias():
    """A zero selection bias and no normalisation is the default top-k."""
    rng = np.random.default_rng(7)
    s = rng.random((30, 64)).astype(np.float32)
    ids0, w0 = oracle.topk(s, 8)
    ids1, w1 = oracle.topk_select(s, np.zeros(64, np.float32), 8)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_array_equal(w0, w1)


def test_topk_select_normalised_weights_sum_to_scale():
    """Normalised weights are proportional to the chosen scores and add up
    to the scale; the bias never enters the weights."""
    rng = np.random.default_rng(8)
    s = rng.random((25, 32)).astype(np.float32)
    b = (rng.standard_normal(32) * 0.3).astype(np.float32)
    ids, w = oracle.topk_select(s, b, 6, normalize=True, scale=2.5)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 2.5, rtol=1e-6)
    chosen = np.take_along_axis(s, ids, axis=1).astype(np.float64)
    np.testing.assert_allclose(w, chosen / chosen.sum(axis=1, keepdims=True) * 2.5, rtol=1e-6)


def test_topk_topp_hand_computed():
    """The top-p cutoff on a worked example (tests/golden/route_topp_hand.json)."""
    with open(os.path.join(GOLD, "route_topp_hand.json")) as fh:
        g = json.load(fh)
    s = np.array([g["scores"]], np.float32)
    ids, w = oracle.topk_select(s, None, g["k"], top_p=g["top_p"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_array_equal(w[0], np.array(g["w_raw"], np.float32))
    ids, w = oracle.topk_select(s, None, g["k"], normalize=True, top_p=g["top_p"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], g["w_normalized"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("p", [0.25, 0.5, 0.625, 0.75, 0.875])
def test_topk_topp_exact_rational(p):
    """With scores that are multiples of 1/64 and a dyadic p every float32 sum
    and product is exact, so the kept slots are exactly the ranked prefix whose
    mass before the slot is below p times the total (checked in rationals)."""
    from fractions import Fraction
    rng = np.random.default_rng(int(p * 1000))
    E, k, N = 16, 6, 50
    s = (rng.integers(1, 64, size=(N, E)).astype(np.float32) / np.float32(64.0))
    ids0, _ = oracle.topk(s, k)
    ids, w = oracle.topk_select(s, None, k, top_p=p)
    for t in range(N):
        ranked = [Fraction(int(round(float(s[t, e]) * 64)), 64) for e in ids0[t]]
        total, before = sum(ranked), Fraction(0)
        for j, e in enumerate(ids0[t]):
            keep = j == 0 or before < Fraction(p).limit_denominator(1 << 20) * total
            before += ranked[j]
            assert ids[t, j] == (e if keep else -1)
            assert w[t, j] == (s[t, e] if keep else 0.0)


@pytest.mark.parametrize("p", [0.0, 1.0, 1.5, -0.5])
def test_topk_topp_off(p):
    rng = np.random.default_rng(3)
    s = rng.random((20, 32)).astype(np.float32)
    a = oracle.topk_select(s, None, 5)
    b = oracle.topk_select(s, None, 5, top_p=p)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_dropped_slot_equals_smaller_k():
    """A slot dropped by the cutoff (id -1) contributes nothing: the layer
    equals the one with that slot removed, and union and counters skip it."""
    cfg = synth.CONFIGS["tiny"]
    spec = cfg.layer
    x, wr, b = synth.tokens(cfg), *synth.router(cfg, 0)
    blocks, shared = synth.expert_pool(cfg, 0), synth.shared_block(cfg, 0)
    ids, w = oracle.topk(oracle.router(x, wr, b), 2)
    ids_d, w_d = ids.copy(), w.copy()
    ids_d[:, 1], w_d[:, 1] = -1, 0.0
    y2 = oracle.expert_forward(blocks, shared, spec.d, spec.f, spec.wbits, spec.group, x, ids_d, w_d)
    y1 = oracle.expert_forward(blocks, shared, spec.d, spec.f, spec.wbits, spec.group, x,
                               ids[:, :1].copy(), w[:, :1].copy())
    np.testing.assert_array_equal(y2, y1)
    u2, off2, _ = oracle.union(ids_d, spec.n_experts)
    u1, off1, _ = oracle.union(ids[:, :1].copy(), spec.n_experts)
    np.testing.assert_array_equal(u2, u1)
    np.testing.assert_array_equal(off2, off1)
    np.testing.assert_array_equal(oracle.hit_count(ids_d, spec.n_experts),
                                  oracle.hit_count(ids[:, :1].copy(), spec.n_experts))


# ---------------------------------------------------------------- union, permutation, counters

@pytest.mark.parametrize("N,k,E", [(1, 1, 4), (5, 3, 8), (17, 4, 16), (64, 8, 256)])
def test_union_perm_counts_brute_force(N, k, E):
    rng = np.random.default_rng(N * 100 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)]).astype(np.int32)
    u, off, perm = oracle.union(ids, E)
    flat = ids.ravel().tolist()
    assert u.tolist() == sorted(set(flat))
    assert off[0] == 0 and off[E] == N * k
    for e in range(E):
        seg = perm[off[e]:off[e + 1]].tolist()
        assert seg == [a for a in range(N * k) if flat[a] == e]
    assert sorted(perm.tolist()) == list(range(N * k))
    c = oracle.hit_count(ids, E)
    assert c.sum() == N * k
    for e in range(E):
        assert c[e] == flat.count(e)
    c2 = oracle.hit_count(ids, E, c.copy())      # counters accumulate
    np.testing.assert_array_equal(c2, 2 * c)


# ---------------------------------------------------------------- dequantisation

@pytest.mark.parametrize("wbits,group", [(4, 32), (4, 128), (4, 0), (8, 0), (8, 64)])
def test_dequant_round_trip(wbits, group):
    """Codes encoded by the test (low nibble = even element) and distinct
    power-of-two scales per group decode exactly to code * scale[c // G]."""
    rng = np.random.default_rng(wbits * 1000 + group)
    rows, cols = 3, 256
    lo, hi = (-8, 8) if wbits == 4 else (-128, 128)
    codes = rng.integers(lo, hi, size=(rows, cols))
    ngr = cols // group if group else 1
    exps = rng.integers(-12, 0, size=(rows, ngr))
    scales = np.ldexp(1.0, exps).astype(np.float32)
    q = pack_codes(codes, wbits)
    for r in range(rows):
        w = oracle.dequant_row(q, scales, r, cols, wbits, group)
        gs = group if group else cols
        expect = np.array([codes[r, c] * math.ldexp(1.0, int(exps[r, c // gs])) for c in range(cols)])
        np.testing.assert_array_equal(w, expect)


# ---------------------------------------------------------------- expert MLP

def _block_from(gc, uc, dc, gs, us, ds, wbits):
    return make_block(gc, uc, dc, gs, us, ds, wbits)


def test_hand_computed_expert():
    g = json.load(open(os.path.join(GOLD, "hand_expert.json")))
    blk = _block_from(g["gate_codes"], g["up_codes"], g["down_codes"], g["gate_scales"],
                      g["up_scales"], g["down_scales"], g["wbits"])
    assert len(blk) == oracle.block_bytes(g["d"], g["f"], g["wbits"], g["group"])
    o = oracle.expert_mlp(blk, g["d"], g["f"], g["wbits"], g["group"], np.array([g["x"]]))
    np.testing.assert_allclose(o[0], g["o"], rtol=1e-15, atol=1e-15)
    pool = blk[None, :]
    y = oracle.expert_forward(pool, None, g["d"], g["f"], g["wbits"], g["group"],
                              np.array([g["x"]], np.float32), np.array([[0]], np.int32),
                              np.array([[g["gate_weight"]]], np.float32))
    np.testing.assert_allclose(y[0], g["y"], rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("wbits,group", [(4, 16), (8, 0)])
def test_expert_exact_integer_case(wbits, group):
    """With gate pre-activations >= 40 (where silu(g) == g exactly in double),
    power-of-two scales and integer inputs, the expert is an exact integer
    computation: compare with int64 matrix products."""
    rng = np.random.default_rng(7 + wbits)
    d, f = 32, 16
    lo, hi = (-8, 8) if wbits == 4 else (-128, 128)
    x_int = rng.integers(-3, 4, size=(2, d))
    x_int[:, 0] = 10                                     # positive lead input
    gc = rng.integers(-1, 2, size=(f, d))
    gc[:, 0] = 7 if wbits == 4 else 100                  # makes every gate row large
    uc = rng.integers(lo, hi, size=(f, d))
    dc = rng.integers(lo, hi, size=(d, f))
    gsh = scales_shape(f, d, group)
    dsh = scales_shape(d, f, group)
    ge = rng.integers(0, 2, size=gsh)
    ue = rng.integers(-3, 0, size=gsh)
    de = rng.integers(-3, 0, size=dsh)
    blk = _block_from(gc, uc, dc, np.ldexp(1.0, ge), np.ldexp(1.0, ue), np.ldexp(1.0, de), wbits)
    gsz = group if group else d
    dsz = group if group else f

    def expand(e, rows, cols, gsize):  # integer exponent per element
        return np.repeat(e, gsize, axis=1)[:, :cols]

    # exact rationals via scaling by 2^8
    Ge = expand(ge, f, d, gsz)
    Ue = expand(ue, f, d, gsz)
    De = expand(de, d, f, dsz)
    g = (gc * (2 ** (Ge + 8))) @ x_int.T                 # = 2^8 * Wg x
    u = (uc * (2 ** (Ue + 8))) @ x_int.T
    assert np.all(g >= 40 * 256)
    h = g * u                                            # = 2^16 * h
    o = (dc * (2 ** (De + 8))) @ h                       # = 2^24 * o
    expect = o.T.astype(np.float64) / 2.0 ** 24
    got = oracle.expert_mlp(blk, d, f, wbits, group, x_int.astype(np.float64))
    np.testing.assert_array_equal(got, expect)


def test_negative_gate_closes_expert():
    """silu(g) -> 0 for g << 0: the expert output vanishes."""
    d, f = 16, 4
    gc = np.full((f, d), -8)
    uc = np.full((f, d), 7)
    dc = np.full((d, f), 7)
    one = lambda r: np.ones((r, 1), np.float32)
    blk = _block_from(gc, uc, dc, one(f), one(f), one(d), 4)
    o = oracle.expert_mlp(blk, d, f, 4, 0, np.ones((1, d)))
    assert np.max(np.abs(o)) < 1e-40


def test_one_hot_input_selects_column():
    """x = e_i reads column i of Wg and Wu only."""
    rng = np.random.default_rng(3)
    d, f = 16, 8
    gc = rng.integers(-8, 8, size=(f, d))
    uc = rng.integers(-8, 8, size=(f, d))
    dc = rng.integers(-8, 8, size=(d, f))
    one = lambda r: np.ones((r, 1), np.float32)
    blk = _block_from(gc, uc, dc, one(f), one(f), one(d), 4)
    for i in (0, 5, 15):
        x = np.zeros((1, d))
        x[0, i] = 1.0
        h = gc[:, i] * expit(gc[:, i].astype(np.float64)) * uc[:, i]   # silu via scipy's expit
        expect = dc @ h
        got = oracle.expert_mlp(blk, d, f, 4, 0, x)[0]
        np.testing.assert_allclose(got, expect, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- layer invariants

def _tiny_layer(seed=0, N=6, k=2, E=8, d=32, f=16, group=16):
    rng = np.random.default_rng(seed)
    pool = np.stack([
        make_block(rng.integers(-8, 8, (f, d)), rng.integers(-8, 8, (f, d)),
                   rng.integers(-8, 8, (d, f)),
                   rng.uniform(0.01, 0.05, (f, d // group)), rng.uniform(0.01, 0.05, (f, d // group)),
                   rng.uniform(0.01, 0.05, (d, f // group)), 4) for _ in range(E + 1)])
    x = rng.standard_normal((N, d)).astype(np.float32)
    wr = (0.3 * rng.standard_normal((E, d))).astype(np.float32)
    return pool[:E], pool[E], x, wr, dict(d=d, f=f, wbits=4, group=group)


def test_zero_gate_equals_dropped_slot():
    pool, shared, x, wr, sh = _tiny_layer()
    ids, w = oracle.topk(oracle.router(x, wr, None), 2)
    w0 = w.copy()
    w0[:, 1] = 0.0
    y2 = oracle.expert_forward(pool, shared, sh["d"], sh["f"], 4, sh["group"], x, ids, w0)
    y1 = oracle.expert_forward(pool, shared, sh["d"], sh["f"], 4, sh["group"], x,
                               ids[:, :1].copy(), w[:, :1].copy())
    np.testing.assert_array_equal(y2, y1)
    # all gates zero leaves the shared expert alone
    yz = oracle.expert_forward(pool, shared, sh["d"], sh["f"], 4, sh["group"], x, ids,
                               np.zeros_like(w))
    ys = oracle.expert_mlp(shared, sh["d"], sh["f"], 4, sh["group"], x.astype(np.float64))
    np.testing.assert_array_equal(yz, ys)


def test_k_equals_E_is_dense_mixture():
    """With k = E every expert is used by every token and the layer is the dense
    sum shared(x) + sum_e s_e * E_e(x)."""
    pool, shared, x, wr, sh = _tiny_layer(seed=4, k=8, E=8)
    E = pool.shape[0]
    out = oracle.layer_step(x, wr, None, E, pool, shared, **sh)
    assert out["union_ids"].tolist() == list(range(E))
    np.testing.assert_array_equal(np.diff(out["offsets"]), np.full(E, x.shape[0]))
    s = out["scores"].astype(np.float64)
    dense = oracle.expert_mlp(shared, sh["d"], sh["f"], 4, sh["group"], x.astype(np.float64))
    for e in range(E):
        dense += s[:, e:e + 1] * oracle.expert_mlp(pool[e], sh["d"], sh["f"], 4, sh["group"],
                                                   x.astype(np.float64))
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


def test_batch_invariance_and_token_permutation():
    pool, shared, x, wr, sh = _tiny_layer(seed=5, N=9)
    full = oracle.layer_step(x, wr, None, 2, pool, shared, **sh)
    sub = [7, 2, 4]
    part = oracle.layer_step(x[sub], wr, None, 2, pool, shared, **sh)
    np.testing.assert_array_equal(part["y"], full["y"][sub])
    np.testing.assert_array_equal(part["ids"], full["ids"][sub])


# ---------------------------------------------------------------- sizes and chaining

def test_block_size_closed_form():
    """3*d*f*bits/8 + 3*d*f/G*4; the int4 GLM-5.2 shape gives the pages' ~19 MB of
    nibbles per expert, and 8 layers x 256 experts give the ~39 GB stack."""
    assert oracle.block_bytes(256, 128, 4, 32) == 61440
    assert oracle.block_bytes(6144, 2048, 4, 128) == 20054016
    assert 3 * 6144 * 2048 // 2 == 18874368
    assert oracle.block_bytes(6144, 2048, 8, 0) == 37789696
    assert abs(8 * 256 * 18874368 / 1e9 - 38.65) < 0.01
    for name, cfg in synth.CONFIGS.items():
        for spec in cfg.layers:
            assert synth.block_bytes(spec) == oracle.block_bytes(spec.d, spec.f, spec.wbits, spec.group)


def test_rms_normalize_closed_form():
    h = np.array([[3.0, 4.0, 0.0, 0.0], [2.0, 2.0, 2.0, 2.0]])
    a = oracle.rms_normalize(h, eps=0.0)
    np.testing.assert_allclose(a[0], np.array([3, 4, 0, 0]) / math.sqrt(25 / 4), rtol=1e-7)
    np.testing.assert_allclose(a[1], np.ones(4), rtol=1e-7)
    a = oracle.rms_normalize(np.full((1, 8), 1e-3), eps=1e-6)
    np.testing.assert_allclose(a[0], np.full(8, 1e-3 / math.sqrt(1e-6 + 1e-6)), rtol=1e-6)


# ---------------------------------------------------------------- Place (LRU cache)

def test_cache_hand_traces():
    """The oracle's per-layer LRU cache reproduces hand-worked traces: hits,
    misses, refusals, pins and prefetches, and the slot contents after each
    call (tests/golden/cache_lru_hand.json)."""
    g = json.load(open(os.path.join(GOLD, "cache_lru_hand.json")))
    for tr in g["traces"]:
        c = oracle.LruCache(tr["n_slots"], tr["n_experts"])
        for st in tr["steps"]:
            before = (c.expert_in.copy(), c.pinned.copy())
            try:
                r = getattr(c, st["op"])(st["ids"])
                r = list(r) if isinstance(r, tuple) else r
            except ValueError:
                r = None
                np.testing.assert_array_equal(c.expert_in, before[0])
                np.testing.assert_array_equal(c.pinned, before[1])
            assert r == st["expect"], st
            assert c.expert_in.tolist() == st["slots"], st
            if "pinned" in st:
                assert c.pinned.tolist() == st["pinned"], st


def _stack_distance_misses(seq, n_slots):
    """Misses of an LRU cache of n_slots on single-expert accesses, from the
    textbook stack-distance property: an access misses exactly when at least
    n_slots distinct other experts were used since its expert's previous
    access, or when there was no previous access."""
    misses = 0
    for i, e in enumerate(seq):
        prev = [j for j in range(i) if seq[j] == e]
        if not prev:
            misses += 1
            continue
        between = set(seq[prev[-1] + 1:i])
        misses += len(between) >= n_slots
    return misses


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cache_matches_lru_stack_distance(seed):
    """One expert per call, no pins: for every cache size, the oracle's misses
    equal the count given by LRU stack distances, computed by brute force."""
    rng = np.random.default_rng(seed)
    E = 12
    # a skewed stream, so that reuse distances of every size occur
    seq = [int(v) for v in rng.zipf(1.3, size=300) % E]
    for C in range(1, E + 1):
        c = oracle.LruCache(C, E)
        misses = sum(c.place([e])[1] for e in seq)
        assert misses == _stack_distance_misses(seq, C), C


def test_cache_large_enough_misses_each_expert_once():
    """A cache with a slot for every expert only takes compulsory misses, for
    unions of any size; every hit or miss is counted once per distinct id."""
    rng = np.random.default_rng(5)
    E = 20
    c = oracle.LruCache(E, E)
    seen, tot_h, tot_m = set(), 0, 0
    for _ in range(50):
        u = rng.integers(0, E, size=int(rng.integers(1, 8))).tolist()
        h, m = c.place(u)
        assert m == len(set(u) - seen)
        assert h + m == len(set(u))
        seen |= set(u)
        tot_h += h
        tot_m += m
    assert tot_m == len(seen)


def test_usage_hottest_brute_force():
    rng = np.random.default_rng(9)
    counts = rng.integers(0, 6, size=40).astype(np.uint64)   # many equal counts
    want = sorted(range(40), key=lambda e: (-int(counts[e]), e))
    for n in (0, 1, 7, 40):
        assert oracle.usage_hottest(counts, n).tolist() == want[:n]
