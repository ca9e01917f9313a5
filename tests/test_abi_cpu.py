"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented codes before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import int4_routed_expert_gemv_amd as moe
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe.so not built")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    probes = declared_functions(os.path.join(ROOT, "include", "moe_probe.h"))
    cache = declared_functions(os.path.join(ROOT, "include", "moe_cache.h"))
    assert set(names) == set(moe.EXPORTED)
    assert set(probes) == set(moe.PROBE_EXPORTED)
    assert set(cache) == set(moe.CACHE_EXPORTED)
    out = subprocess.check_output(["nm", "-D", "--defined-only", moe.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names + cache:
        assert n in exported, n
        assert hasattr(moe.lib(), n)
    # the measurement probes live in their own library, not in the product one
    out = subprocess.check_output(["nm", "-D", "--defined-only", moe.PROBE_LIB_PATH], text=True)
    probe_exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in probes:
        assert n in probe_exported and n not in exported, n
        assert hasattr(moe.probe_lib(), n)


def test_every_launched_kernel_has_gfx950_code():
    """Each kernel the host code can launch has a descriptor in the library's
    code object (host and device passes built from one version of a source)."""
    from int4_routed_expert_gemv_amd import build
    for path in (moe.LIB_PATH, moe.PROBE_LIB_PATH):
        stubs = {m.decode() for m in build._STUB.findall(open(path, "rb").read())}
        assert stubs, path
        assert all(build._kernel_of_stub(s) for s in stubs), path
        assert build.kernels_without_code(path) == [], path


def test_probe_argument_checks():
    L = moe.probe_lib()
    # size not a multiple of 1024, bad batch, bad workgroup, sink too small, misaligned
    assert L.moe_probe_stream_read(FAKE, 1000, 3, 4, FAKE, 1 << 20, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_stream_read(FAKE, 1 << 20, 5, 4, FAKE, 1 << 20, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_stream_read(FAKE, 1 << 20, 3, 17, FAKE, 1 << 20, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_stream_read(FAKE, 1 << 20, 3, 4, FAKE, 10, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_stream_read(FAKE + 4, 1 << 20, 3, 4, FAKE, 1 << 20, None, None, None) == moe.MOE_EALIGN
    assert L.moe_probe_stream_read(None, 1 << 20, 3, 4, FAKE, 1 << 20, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_mfma_f16(None, 4, 4, None, None, None) == moe.MOE_EINVAL
    assert L.moe_probe_mfma_f16(FAKE, 0, 4, None, None, None) == moe.MOE_EINVAL


def _pool(d=256, f=128, E=16, wbits=4, group=32, pool=4096, stride=None, shared=None):
    bb = moe.block_bytes(d, f, wbits, group)
    stride = stride if stride is not None else (bb + 255) // 256 * 256
    return moe.PoolDesc(d, f, E, wbits, group, pool, stride, shared)


FAKE = 1 << 20  # aligned non-null address: never dereferenced, every call below fails first


def test_route_union_argument_checks():
    """moe_route_union makes every check of the three calls it stands for
    before launching anything, on both sides of the one-workgroup tail size."""
    L = moe.lib()
    big = 1 << 30

    def call(x=FAKE, N=4, d=256, wr=FAKE, E=16, k=1, ids=FAKE, w=FAKE, uid=FAKE, nu=FAKE,
             off=FAKE, perm=FAKE, cnt=None, ws=FAKE, wsb=big):
        return L.moe_route_union(x, N, d, wr, None, E, k, ids, w, uid, nu, off, perm, cnt, ws,
                                 wsb, None)

    for N in (4, 40):
        assert call(N=N, k=0) == moe.MOE_EINVAL
        assert call(N=N, k=17) == moe.MOE_EINVAL
        assert call(N=N, E=2000, k=8) == moe.MOE_EINVAL
        assert call(N=-1) == moe.MOE_EINVAL
        assert call(N=N, x=None) == moe.MOE_EINVAL
        assert call(N=N, uid=None) == moe.MOE_EINVAL
        assert call(N=N, nu=None) == moe.MOE_EINVAL
        assert call(N=N, off=None) == moe.MOE_EINVAL
        assert call(N=N, perm=None) == moe.MOE_EINVAL
        assert call(N=N, d=48) == moe.MOE_ESHAPE
        assert call(N=N, wsb=10) == moe.MOE_EWORKSPACE
        assert call(N=N, ws=None) == moe.MOE_EWORKSPACE
        assert call(N=N, x=FAKE + 4) == moe.MOE_EALIGN
        assert call(N=N, cnt=FAKE + 4) == moe.MOE_EALIGN
        assert call(N=N, ws=FAKE + 16) == moe.MOE_EALIGN
    assert call(N=0, x=None, ids=None) == moe.MOE_OK  # nothing to do


@pytest.mark.parametrize("sel,norm,scale,top_p", [
    (2, 0, 1.0, 0.0), (-1, 0, 1.0, 0.0), (0, 3, 1.0, 0.0), (1, 1, 0.0, 0.0), (1, 1, -2.0, 0.0),
    (0, 0, float("nan"), 0.0), (0, 1, float("inf"), 0.0), (0, 0, 1.0, float("nan")),
    (0, 0, 1.0, -0.25), (1, 0, 1.0, float("inf"))])
def test_route_options_are_checked_before_launch(sel, norm, scale, top_p):
    """The _ex calls reject a bad router option with MOE_EINVAL (nothing is
    enqueued, so fake device pointers are never touched)."""
    L = moe.lib()
    big = 1 << 30
    opt = ctypes.byref(moe.RouteOptions(sel, norm, scale, top_p))
    assert L.moe_route_topk_ex(FAKE, 4, 256, FAKE, FAKE, 16, 2, FAKE, FAKE, FAKE, big, None,
                               opt) == moe.MOE_EINVAL
    for N in (4, 40):
        assert L.moe_route_union_ex(FAKE, N, 256, FAKE, FAKE, 16, 2, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None, FAKE, big, None, opt) == moe.MOE_EINVAL


def test_route_options_misaligned_bias_and_empty_batch():
    L = moe.lib()
    big = 1 << 30
    opt = ctypes.byref(moe.RouteOptions(1, 1, 2.5))
    assert L.moe_route_union_ex(FAKE, 4, 256, FAKE, FAKE + 2, 16, 2, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, FAKE, big, None, opt) == moe.MOE_EALIGN
    assert L.moe_route_union_ex(None, 0, 256, None, None, 16, 2, None, None, None, None, None,
                                None, None, None, 0, None, opt) == moe.MOE_OK


def test_route_topk_argument_checks():
    L = moe.lib()
    ws = FAKE
    big = 1 << 30
    # k out of range
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 0, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 17, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 64, 33, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 2000, 8, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    # negative tokens, null pointers, workspace, alignment
    assert L.moe_route_topk(FAKE, -1, 256, FAKE, None, 16, 1, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(None, 4, 256, FAKE, None, 16, 1, FAKE, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 1, None, FAKE, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 1, FAKE, FAKE, ws, 10, None) == moe.MOE_EWORKSPACE
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 1, FAKE, FAKE, None, big, None) == moe.MOE_EWORKSPACE
    assert L.moe_route_topk(FAKE + 4, 4, 256, FAKE, None, 16, 1, FAKE, FAKE, ws, big, None) == moe.MOE_EALIGN
    assert L.moe_route_topk(FAKE, 4, 256, FAKE, None, 16, 1, FAKE, FAKE, ws + 16, big, None) == moe.MOE_EALIGN
    assert L.moe_route_topk(FAKE, 4, 250, FAKE, None, 16, 1, FAKE, FAKE, ws, big, None) == moe.MOE_ESHAPE
    assert L.moe_route_topk(FAKE, 4, 48, FAKE, None, 16, 1, FAKE, FAKE, ws, big, None) == moe.MOE_ESHAPE
    # zero tokens: success, nothing touched (even with null pointers)
    assert L.moe_route_topk(None, 0, 256, None, None, 16, 1, None, None, None, 0, None) == moe.MOE_OK


def test_union_and_hit_count_argument_checks():
    L = moe.lib()
    assert L.moe_union(FAKE, 4, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_union(FAKE, 4, 2, 0, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_union(FAKE, -4, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_union(FAKE, 4, 2, 16, FAKE, None, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_union(None, 0, 2, 16, None, None, None, None, None) == moe.MOE_OK
    assert L.moe_hit_count(FAKE, 4, 3, 2, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_hit_count(FAKE, 4, 1, 2, None, None) == moe.MOE_EINVAL
    assert L.moe_hit_count(FAKE, 4, 1, 2, FAKE + 4, None) == moe.MOE_EALIGN
    assert L.moe_hit_count(None, 0, 1, 2, None, None) == moe.MOE_OK


def _fwd(pool, N=4, k=1, ws=FAKE, wsb=1 << 30, x=FAKE, y=FAKE):
    return moe.lib().moe_expert_forward(ctypes.byref(pool), x, N, k, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        y, ws, wsb, None)


def test_expert_forward_argument_checks():
    assert _fwd(_pool(wbits=3)) == moe.MOE_EINVAL
    assert _fwd(_pool(d=250)) == moe.MOE_ESHAPE            # not a multiple of 128
    assert _fwd(_pool(d=160)) == moe.MOE_ESHAPE            # a multiple of 32, not of 128
    assert _fwd(_pool(f=192)) == moe.MOE_ESHAPE
    assert _fwd(_pool(d=16384 + 128)) == moe.MOE_ESHAPE    # beyond the largest dimension
    assert _fwd(_pool(group=48)) == moe.MOE_ESHAPE         # group not a multiple of 32
    assert _fwd(_pool(group=96)) == moe.MOE_ESHAPE         # group does not divide d or f
    assert _fwd(_pool(E=0)) == moe.MOE_EINVAL
    assert _fwd(_pool(E=2000)) == moe.MOE_EINVAL
    assert _fwd(_pool(), k=17) == moe.MOE_EINVAL
    assert _fwd(_pool(pool=None)) == moe.MOE_EINVAL
    assert _fwd(_pool(pool=FAKE + 64)) == moe.MOE_EALIGN
    assert _fwd(_pool(shared=FAKE + 64)) == moe.MOE_EALIGN
    assert _fwd(_pool(stride=61440 + 16)) == moe.MOE_EALIGN
    assert _fwd(_pool(stride=256)) == moe.MOE_ESHAPE       # stride smaller than a block
    assert _fwd(_pool(), wsb=100) == moe.MOE_EWORKSPACE
    assert _fwd(_pool(), ws=None) == moe.MOE_EWORKSPACE
    assert _fwd(_pool(), ws=FAKE + 32) == moe.MOE_EALIGN
    assert _fwd(_pool(), x=FAKE + 4) == moe.MOE_EALIGN
    assert _fwd(_pool(), N=-1) == moe.MOE_EINVAL
    assert _fwd(_pool(), N=0, x=None, y=None, ws=None, wsb=0) == moe.MOE_OK
    assert moe.lib().moe_residual_rmsnorm(FAKE, None, FAKE, 2, 0, 1e-6, None) == moe.MOE_EINVAL
    assert moe.lib().moe_residual_rmsnorm(FAKE, None, FAKE, 2, 8, -1.0, None) == moe.MOE_EINVAL
    assert moe.lib().moe_residual_rmsnorm(FAKE, None, FAKE, 0, 8, 1e-6, None) == moe.MOE_OK


def test_sizes():
    for name, cfg in synth.CONFIGS.items():
        for spec in cfg.layers:
            assert moe.block_bytes(spec.d, spec.f, spec.wbits, spec.group) == synth.block_bytes(spec)
    assert moe.block_bytes(6144, 2048, 4, 128) == 20054016
    assert moe.block_bytes(6144, 2048, 8, 0) == 37789696
    p = _pool(d=6144, f=2048, E=256, group=128, shared=FAKE)
    N, k = 64, 8
    A = N * k
    ws = moe.forward_workspace_size(p, N, k)
    # hidden [A+N][f] and expert outputs [A+N][d] in float32 dominate, plus the
    # float16 input [N][d] and hidden [A+N][f] of the matrix-core passes
    big = (A + N) * (2048 + 6144) * 4 + N * 6144 * 2 + (A + N) * 2048 * 2
    assert big <= ws < big + 2 * 1024 * 1024
    # scores, or router partial sums over at most 16 slices of the contraction
    assert N * 256 * 4 <= moe.route_workspace_size(N, 256) <= 16 * N * 256 * 4
    assert moe.route_workspace_size(1, 256) == 256 * 4
    assert moe.workspace_size(p, N, k) == max(ws, moe.route_workspace_size(N, 256))
    assert moe.forward_workspace_size(_pool(wbits=5), N, k) == 0
    # without a shared expert there are no shared rows
    p0 = _pool(d=6144, f=2048, E=256, group=128)
    assert moe.forward_workspace_size(p0, N, k) < ws - N * (2048 + 6144) * 4 - N * 2048 * 2 + 4096


def _units(codes, R, K, wbits):
    """The documented device arrangement of one canonical code matrix:
    1 KB units of 16 rows x (128 int4 or 64 int8) columns, slot r + 16 q of
    unit (rt, kb) holding the 16 bytes of row 16 rt + r at quarter q."""
    rb = K * wbits // 8
    m = codes.reshape(R // 16, 16, K // (512 // wbits), 4, 16)   # rt, r, kb, q, byte
    return m.transpose(0, 2, 3, 1, 4).reshape(R * rb)


def _scale_units(sc, R, ng):
    return sc.reshape(R // 16, 16, ng).transpose(0, 2, 1).reshape(R * ng)


@pytest.mark.parametrize("wbits,d,f,group", [(4, 256, 128, 32), (4, 384, 256, 128),
                                              (8, 192, 128, 0), (8, 128, 64, 32)])
def test_pack_expert_unit_layout(wbits, d, f, group):
    """moe_pack_expert against the layout the header documents, on random
    bytes (so every byte's destination is checked)."""
    nb = moe.block_bytes(d, f, wbits, group)
    rng = np.random.default_rng(wbits * 1000 + d + f + group)
    blk = rng.integers(0, 256, nb, dtype=np.uint8)
    out = moe.pack_expert(blk.copy(), _pool(d=d, f=f, wbits=wbits, group=group))
    flip = 0x88 if wbits == 4 else 0x80
    q = d * f * wbits // 8
    exp = np.empty_like(blk)
    for off, R, K in ((0, f, d), (q, f, d), (2 * q, d, f)):
        exp[off:off + q] = _units(blk[off:off + q] ^ flip, R, K, wbits)
    sc = blk[3 * q:].view(np.float32)
    ng_gu, ng_dn = (d // group, f // group) if group else (1, 1)
    s_exp = np.empty_like(sc)
    o = 0
    for R, ng in ((f, ng_gu), (f, ng_gu), (d, ng_dn)):
        s_exp[o:o + R * ng] = _scale_units(sc[o:o + R * ng], R, ng)
        o += R * ng
    exp[3 * q:] = s_exp.view(np.uint8)
    np.testing.assert_array_equal(out, exp)
    # in place gives the same
    same = blk.copy()
    moe.pack_expert(same, _pool(d=d, f=f, wbits=wbits, group=group), same)
    np.testing.assert_array_equal(same, exp)
    with pytest.raises(moe.MoeError):
        moe.pack_expert(blk, _pool(d=250))


def test_strerror():
    for s in range(-5, 1):
        assert moe.strerror(s)
    assert "workspace" in moe.strerror(moe.MOE_EWORKSPACE)


def test_cache_argument_checks():
    """moe_cache_create / moe_cache_place reject bad arguments before any HIP call."""
    L = moe.lib()
    h = ctypes.c_void_p()
    big = 1 << 20
    assert L.moe_cache_create(16, 4, 1000, 1024, FAKE, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_cache_create(0, 1, 1000, 1024, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(2000, 4, 1000, 1024, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(16, 0, 1000, 1024, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(16, 17, 1000, 1024, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(16, 4, 2000, 1024, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(16, 4, 1000, 1024, None, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EINVAL
    assert L.moe_cache_create(16, 4, 1000, 1000, FAKE, FAKE, FAKE, ctypes.byref(h)) == moe.MOE_EALIGN
    assert L.moe_cache_create(16, 4, 1000, 1024, FAKE, FAKE + 16, FAKE, ctypes.byref(h)) == moe.MOE_EALIGN
    assert not h.value
    assert L.moe_cache_place(None, FAKE, 1, None, None, None) == moe.MOE_EINVAL
    assert L.moe_cache_stats(None, None, None) == moe.MOE_EINVAL
    del big


# ---------------------------------------------------------------- usage file and hottest experts

def test_usage_file_round_trip_and_errors(tmp_path):
    """moe_usage_write / moe_usage_read: the counters come back exactly;
    other dimensions, a foreign or damaged file and a missing one are
    errors that leave the output untouched."""
    rng = np.random.default_rng(1)
    c = rng.integers(0, 1 << 40, size=(9, 256)).astype(np.uint64)
    c[0, 0] = np.uint64((1 << 64) - 1)
    path = str(tmp_path / "layers.usage")
    moe.usage_write(path, c)
    np.testing.assert_array_equal(moe.usage_read(path, 9, 256), c)
    assert os.path.getsize(path) == 8 + 12 + 9 * 256 * 8
    with pytest.raises(moe.MoeError) as e:
        moe.usage_read(path, 8, 256)
    assert e.value.status == moe.MOE_ESHAPE
    raw = open(path, "rb").read()
    for bad in (b"NOTUSAGE" + raw[8:], raw[:-1], raw + b"\0", raw[:10]):
        (tmp_path / "bad").write_bytes(bad)
        with pytest.raises(moe.MoeError) as e:
            moe.usage_read(str(tmp_path / "bad"), 9, 256)
        assert e.value.status == moe.MOE_EIO
    with pytest.raises(moe.MoeError) as e:
        moe.usage_read(str(tmp_path / "missing"), 9, 256)
    assert e.value.status == moe.MOE_EIO
    L = moe.lib()
    out = np.full((9, 256), 7, np.uint64)
    assert L.moe_usage_read(os.fsencode(str(tmp_path / "bad")), out.ctypes.data, 9, 256) == moe.MOE_EIO
    assert np.all(out == 7)
    assert L.moe_usage_write(None, c.ctypes.data, 9, 256) == moe.MOE_EINVAL
    assert L.moe_usage_write(os.fsencode(path), c.ctypes.data, 0, 256) == moe.MOE_EINVAL


def test_usage_hottest_ranks_by_hits_then_id():
    rng = np.random.default_rng(2)
    c = rng.integers(0, 6, size=300).astype(np.uint64)   # many equal counts
    for n in (0, 1, 17, 300):
        got = moe.usage_hottest(c, n)
        ref = sorted(range(300), key=lambda e: (-int(c[e]), e))[:n]
        assert got.tolist() == ref
    L = moe.lib()
    ids = np.empty(4, np.int32)
    assert L.moe_usage_hottest(c.ctypes.data, 300, 301, ids.ctypes.data) == moe.MOE_EINVAL
    assert L.moe_usage_hottest(None, 300, 4, ids.ctypes.data) == moe.MOE_EINVAL


def test_cache_calls_reject_a_null_cache():
    L = moe.lib()
    ids = np.zeros(4, np.int32)
    for name in ("moe_cache_pin", "moe_cache_prefetch"):
        assert getattr(L, name)(None, ids.ctypes.data, 4, None, None, None) == moe.MOE_EINVAL
    assert L.moe_cache_resident(None, None, None) == moe.MOE_EINVAL


def _step(pool, N=1, k=1, d=None, ws=FAKE, wsb=1 << 30, x=FAKE, wr=FAKE, y=FAKE):
    d = pool.d_model if d is None else d
    return moe.lib().moe_layer_step(ctypes.byref(pool), x, N, d, wr, None, k, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, None, y, ws, wsb, None, None)


def test_layer_step_argument_checks():
    """moe_layer_step makes every check of moe_route_union and
    moe_expert_forward before launching anything."""
    p = _pool()
    need = moe.layer_step_workspace_size(p, 1, 1)
    assert need == moe.route_workspace_size(1, 16) + moe.forward_workspace_size(p, 1, 1)
    assert moe.layer_step_workspace_size(_pool(wbits=3), 1, 1) == 0
    assert _step(p, wsb=need - 1) == moe.MOE_EWORKSPACE
    assert _step(p, ws=None) == moe.MOE_EWORKSPACE
    assert _step(p, d=512) == moe.MOE_ESHAPE                  # d_model differs from the pool's
    assert _step(p, k=17) == moe.MOE_EINVAL                   # k above n_experts
    assert _step(p, k=0) == moe.MOE_EINVAL
    assert _step(p, x=None) == moe.MOE_EINVAL
    assert _step(p, wr=None) == moe.MOE_EINVAL
    assert _step(p, y=None) == moe.MOE_EINVAL
    assert _step(p, x=FAKE + 4) == moe.MOE_EALIGN
    assert _step(p, ws=FAKE + 64, wsb=1 << 30) == moe.MOE_EALIGN
    assert _step(_pool(d=250), d=250) == moe.MOE_ESHAPE       # not a multiple of 128
    assert _step(p, N=-1) == moe.MOE_EINVAL
    assert _step(p, N=0) == moe.MOE_OK                        # an empty batch is a no-op
    assert moe.lib().moe_layer_step(None, FAKE, 1, 256, FAKE, None, 1, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None,
                                    None) == moe.MOE_EINVAL


def test_layer_step_noalloc_rejects_oversize_steps_before_any_hip_call():
    """moe_layer_step_noalloc: a step whose workspace exceeds the library's
    array (MOE_SCRATCH_BYTES) and a missing pool are refused on the host,
    so this runs without a GPU."""
    assert moe.MOE_SCRATCH_BYTES == 64 << 20
    glm = _pool(d=6144, f=2048, E=256, group=128)
    assert moe.layer_step_workspace_size(glm, 128, 8) <= moe.MOE_SCRATCH_BYTES
    assert moe.layer_step_workspace_size(glm, 256, 8) > moe.MOE_SCRATCH_BYTES
    L = moe.lib()
    args = (FAKE, 256, 6144, FAKE, None, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
            None)
    assert L.moe_layer_step_noalloc(ctypes.byref(glm), *args) == moe.MOE_EWORKSPACE
    assert L.moe_layer_step_noalloc(None, *args) == moe.MOE_EINVAL


def test_stack_forward_argument_checks():
    """moe_stack_forward: every layer's checks before anything is enqueued."""
    L = moe.lib()
    p = _pool()
    layers = moe.layer_descs([(p, None, None, None), (p, None, None, None)])
    for ld in layers:
        ld.w_router = FAKE
    need = moe.stack_workspace_size(layers, 4, 2)
    assert need > moe.layer_step_workspace_size(p, 4, 2)   # one layer step's, reused
    assert L.moe_stack_forward(None, 1, 4, 2, 1e-6, FAKE, None, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_stack_forward(layers, 0, 4, 2, 1e-6, FAKE, None, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_stack_forward(layers, 2, 4, 2, -1.0, FAKE, None, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_stack_forward(layers, 2, 4, 2, 1e-6, FAKE, None, FAKE, need - 1,
                               None) == moe.MOE_EWORKSPACE
    assert L.moe_stack_forward(layers, 2, 4, 2, 1e-6, None, None, FAKE, need, None) == moe.MOE_EINVAL
    assert L.moe_stack_forward(layers, 2, 4, 2, 1e-6, FAKE + 4, None, FAKE, need,
                               None) == moe.MOE_EALIGN
    assert L.moe_stack_forward(layers, 2, 4, 17, 1e-6, FAKE, None, FAKE, 1 << 30,
                               None) == moe.MOE_EINVAL            # k above n_experts
    assert L.moe_stack_forward(layers, 2, 0, 2, 1e-6, None, None, None, 0, None) == moe.MOE_OK
    layers[1].w_router = None                                    # the second layer's router
    assert L.moe_stack_forward(layers, 2, 4, 2, 1e-6, FAKE, None, FAKE, need, None) == moe.MOE_EINVAL
    layers[1].w_router = FAKE
    layers[1].pool = _pool(d=512)                                # layers of different widths
    assert moe.stack_workspace_size(layers, 4, 2) == 0
    assert L.moe_stack_forward(layers, 2, 4, 2, 1e-6, FAKE, None, FAKE, 1 << 30,
                               None) == moe.MOE_ESHAPE
