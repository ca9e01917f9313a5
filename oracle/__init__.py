"""CPU oracle of the routed-expert layer step (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never does. The arithmetic lives in ``oracle.c`` (plain C99,
double precision, OpenMP over independent rows). This module only marshals
numpy arrays.

Pages followed: the Colibri pages "Public Colibri Observation and Revision
Ledger" (section "Exact Architecture and Data-Flow Reconstruction": sigmoid
router with n_group=1 and float32 gate parameters, three-matrix expert MLPs,
an always-on shared expert, the Route/Union/Place/Overlap/Learn stages and the
per-expert hit counters) and the Colibri README ("Get started": group-scaled
int4 experts; "Speculative decoding, honestly": the int8 draft head).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# a test that plants mistakes in a copy of the oracle loads that copy instead
_LOAD_PATH = os.environ.get("ORACLE_LIB_OVERRIDE", _LIB_PATH)
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LOAD_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.oracle_block_bytes.restype = sz
        L.oracle_block_bytes.argtypes = [i32] * 4
        L.oracle_dequant_row.argtypes = [vp, vp, i32, i32, i32, i32, vp]
        L.oracle_router.argtypes = [vp, i32, i32, vp, vp, i32, vp, vp]
        L.oracle_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_topk_select.argtypes = [vp, vp, i32, i32, i32, i32, ctypes.c_double,
                                         ctypes.c_float, vp, vp]
        L.oracle_union.restype = i32
        L.oracle_union.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_hit_count.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_expert_mlp.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp]
        L.oracle_expert_forward.restype = i32
        L.oracle_expert_forward.argtypes = [vp, sz, i32, vp, i32, i32, i32, i32,
                                            vp, i32, i32, vp, vp, vp]
        L.oracle_rms_normalize.argtypes = [vp, i32, i32, ctypes.c_double, vp]
        u64p = vp
        L.oracle_cache_place.restype = i32
        L.oracle_cache_place.argtypes = [i32, i32, vp, u64p, vp, u64p, vp, i32, vp, vp]
        L.oracle_cache_pin.restype = i32
        L.oracle_cache_pin.argtypes = [i32, i32, vp, u64p, vp, u64p, vp, i32, vp]
        L.oracle_cache_prefetch.argtypes = [i32, i32, vp, u64p, vp, u64p, vp, i32, vp]
        L.oracle_usage_hottest.argtypes = [vp, i32, i32, vp]
        L.oracle_threads.restype = i32
        L.oracle_threads.argtypes = []
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def threads() -> int:
    """OpenMP threads the oracle's parallel loops run with on this host."""
    return int(lib().oracle_threads())


def block_bytes(d, f, wbits, group) -> int:
    return int(lib().oracle_block_bytes(d, f, wbits, group))


def dequant_row(q, scales, r, cols, wbits, group) -> np.ndarray:
    q, qp = _c(q, np.uint8)
    s, sp = _c(scales, np.float32)
    out = np.empty(cols, np.float64)
    lib().oracle_dequant_row(qp, sp, r, cols, wbits, group, out.ctypes.data)
    return out


def router(x, w_router, b_router=None, return_logits=False):
    """Scores s[N][E] (float32) = sigmoid(Wr x + b)."""
    x, xp = _c(x, np.float32)
    wr, wp = _c(w_router, np.float32)
    N, d = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == d
    bp = None
    if b_router is not None:
        b, bp = _c(b_router, np.float32)
    s = np.empty((N, E), np.float32)
    logits = np.empty((N, E), np.float64) if return_logits else None
    lib().oracle_router(xp, N, d, wp, bp, E, s.ctypes.data,
                        logits.ctypes.data if return_logits else None)
    return (s, logits) if return_logits else s


def topk(scores, k):
    s, sp = _c(scores, np.float32)
    N, E = s.shape
    ids = np.empty((N, k), np.int32)
    w = np.empty((N, k), np.float32)
    lib().oracle_topk(sp, N, E, k, ids.ctypes.data, w.ctypes.data)
    return ids, w


def topk_select(scores, b_sel, k, normalize=False, scale=1.0, top_p=0.0):
    """Router variant: the bias b_sel only steers the selection (key = s + b
    in float32); weights are the unbiased scores, optionally divided by their
    sum over the chosen k, times scale. scores: unbiased sigmoid scores [N][E]
    (router(x, Wr) with no bias); b_sel None: no selection bias. top_p in
    (0, 1): ranked slots past that fraction of the chosen score mass get id -1
    and weight 0."""
    s, sp = _c(scores, np.float32)
    N, E = s.shape
    bp = None
    if b_sel is not None:
        b, bp = _c(b_sel, np.float32)
        assert b.shape == (E,)
    ids = np.empty((N, k), np.int32)
    w = np.empty((N, k), np.float32)
    lib().oracle_topk_select(sp, bp, N, E, k, 1 if normalize else 0, float(scale),
                             float(top_p), ids.ctypes.data, w.ctypes.data)
    return ids, w


def union(ids, n_experts):
    """(union_ids[:n_union], offsets[E+1], perm[N*k])."""
    ids, ip = _c(ids, np.int32)
    N, k = ids.shape
    u = np.empty(n_experts, np.int32)
    off = np.empty(n_experts + 1, np.int32)
    perm = np.empty(N * k, np.int32)
    n = lib().oracle_union(ip, N, k, n_experts, u.ctypes.data, off.ctypes.data, perm.ctypes.data)
    return u[:n].copy(), off, perm


def hit_count(ids, n_experts, counters=None):
    ids, ip = _c(ids, np.int32)
    N, k = ids.shape
    if counters is None:
        counters = np.zeros(n_experts, np.uint64)
    assert counters.dtype == np.uint64 and counters.flags["C_CONTIGUOUS"]
    lib().oracle_hit_count(ip, N, k, n_experts, counters.ctypes.data)
    return counters


def expert_mlp(block, d, f, wbits, group, X):
    """O[T][d] (double) for one expert block on token vectors X[T][d]."""
    blk, bp = _c(block, np.uint8)
    X, xp = _c(np.atleast_2d(X), np.float64)
    T = X.shape[0]
    O = np.empty((T, d), np.float64)
    lib().oracle_expert_mlp(bp, d, f, wbits, group, xp, T, O.ctypes.data)
    return O


def expert_forward(pool, shared, d, f, wbits, group, x, ids, w):
    """y[N][d] (double) = shared(x) + sum_j w[t][j] * expert_{ids[t][j]}(x)."""
    pool = np.ascontiguousarray(pool, np.uint8)
    E, stride = pool.shape
    shp = None
    if shared is not None:
        shared, shp = _c(shared, np.uint8)
    x, xp = _c(x, np.float32)
    ids, ip = _c(ids, np.int32)
    w, wp = _c(w, np.float32)
    N, k = ids.shape
    y = np.empty((N, d), np.float64)
    rc = lib().oracle_expert_forward(pool.ctypes.data, stride, E, shp, d, f, wbits, group,
                                     xp, N, k, ip, wp, y.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_expert_forward: expert id out of range")
    return y


def rms_normalize(h, eps=1e-6):
    h, hp = _c(h, np.float64)
    N, d = h.shape
    a = np.empty((N, d), np.float32)
    lib().oracle_rms_normalize(hp, N, d, eps, a.ctypes.data)
    return a


def layer_step(x, w_router, b_router, k, pool, shared, d, f, wbits, group, counters=None):
    """The whole layer step: route, top-k, union, hit counters, experts, combine."""
    E = w_router.shape[0]
    s = router(x, w_router, b_router)
    ids, w = topk(s, k)
    u, off, perm = union(ids, E)
    counters = hit_count(ids, E, counters)
    y = expert_forward(pool, shared, d, f, wbits, group, x, ids, w)
    return dict(scores=s, ids=ids, w=w, union_ids=u, offsets=off, perm=perm,
                counters=counters, y=y)


class LruCache:
    """Place stage: a per-layer LRU cache of n_slots expert blocks (the
    arithmetic is oracle_cache_* in oracle.c; this class only holds the
    state arrays). place/pin/prefetch return (hits, misses), misses and
    copies; place and pin raise ValueError when refused (state unchanged)."""

    def __init__(self, n_slots, n_experts):
        self.n_slots, self.n_experts = n_slots, n_experts
        self.expert_in = np.full(n_slots, -1, np.int32)
        self.last_use = np.zeros(n_slots, np.uint64)
        self.pinned = np.zeros(n_slots, np.int32)
        self.clock = np.zeros(1, np.uint64)

    def _args(self):
        return (self.n_slots, self.n_experts, self.expert_in.ctypes.data,
                self.last_use.ctypes.data, self.pinned.ctypes.data, self.clock.ctypes.data)

    def place(self, ids):
        ids = np.ascontiguousarray(ids, np.int32)
        h, m = np.zeros(1, np.int32), np.zeros(1, np.int32)
        if lib().oracle_cache_place(*self._args(), ids.ctypes.data, ids.size, h.ctypes.data,
                                    m.ctypes.data):
            raise ValueError("union larger than the unpinned slots")
        return int(h[0]), int(m[0])

    def pin(self, ids):
        ids = np.ascontiguousarray(ids, np.int32)
        m = np.zeros(1, np.int32)
        if lib().oracle_cache_pin(*self._args(), ids.ctypes.data, ids.size, m.ctypes.data):
            raise ValueError("pin set larger than the slots")
        return int(m[0])

    def prefetch(self, ids):
        ids = np.ascontiguousarray(ids, np.int32)
        c = np.zeros(1, np.int32)
        lib().oracle_cache_prefetch(*self._args(), ids.ctypes.data, ids.size, c.ctypes.data)
        return int(c[0])

    def slot_of(self):
        """[n_experts] slot of each expert, -1 when not resident."""
        so = np.full(self.n_experts, -1, np.int32)
        for s, e in enumerate(self.expert_in):
            if e >= 0:
                so[e] = s
        return so


def usage_hottest(counters, n):
    c = np.ascontiguousarray(counters, np.uint64)
    ids = np.empty(n, np.int32)
    lib().oracle_usage_hottest(c.ctypes.data, c.size, n, ids.ctypes.data)
    return ids
