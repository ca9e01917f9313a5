"""Python binding of the routed-expert layer step (libmoe.so, include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI. PyTorch provides device memory and the stream. If the
library has not been built, the binding raises. There is no fallback path.

The layer (after the Colibri pages, "Public Colibri Observation and Revision
Ledger", section "Exact Architecture and Data-Flow Reconstruction"):
  route_topk      float32 sigmoid router over all experts (n_group = 1) + top-k
  union           batch union of the routed experts + token->expert permutation
  hit_count       per-expert hit counters (the Learn stage)
  expert_forward  int4/int8 SwiGLU experts over the union + the shared expert,
                  combined by gate weight
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
# measurement probes (include/moe_probe.h): a library of their own, loaded by
# the benchmark only
PROBE_LIB_PATH = os.path.join(_HERE, "libmoe_probe.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP, MOE_EIO = (
    0, -1, -2, -3, -4, -5, -6)
MOE_MAX_K = 32
MOE_MAX_EXPERTS = 1024
MOE_ALIGN = 256

EXPORTED = [
    "moe_route_topk", "moe_route_topk_ex", "moe_union", "moe_route_union", "moe_route_union_ex",
    "moe_expert_forward", "moe_expert_forward_ex",
    "moe_hit_count", "moe_residual_rmsnorm", "moe_route_workspace_size", "moe_forward_workspace_size",
    "moe_workspace_size", "moe_block_bytes", "moe_pack_expert", "moe_strerror",
    "moe_layer_step", "moe_layer_step_workspace_size", "moe_layer_step_noalloc",
    "moe_stack_forward", "moe_stack_workspace_size",
]
MOE_SCRATCH_BYTES = 64 << 20  # the workspace array of moe_layer_step_noalloc, per GPU


# measured-ceiling probes (include/moe_probe.h), not part of the layer step
PROBE_EXPORTED = ["moe_probe_stream_read", "moe_probe_mfma_f16"]
# the expert cache of the Place stage (include/moe_cache.h)
CACHE_EXPORTED = ["moe_cache_create", "moe_cache_destroy", "moe_cache_place", "moe_cache_forward",
                  "moe_cache_stats",
                  "moe_cache_pin", "moe_cache_prefetch", "moe_cache_resident", "moe_usage_write",
                  "moe_usage_read", "moe_usage_hottest"]


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {strerror(status)} (status {status})")


class ForwardOptions(ctypes.Structure):
    """struct moe_forward_options (HIP event handles, NULL = not taken)"""
    _fields_ = [("gateup_start", ctypes.c_void_p), ("gateup_end", ctypes.c_void_p),
                ("down_start", ctypes.c_void_p), ("down_end", ctypes.c_void_p),
                ("mfma_gateup_start", ctypes.c_void_p), ("mfma_gateup_end", ctypes.c_void_p),
                ("mfma_down_start", ctypes.c_void_p), ("mfma_down_end", ctypes.c_void_p),
                ("small_gateup_start", ctypes.c_void_p), ("small_gateup_end", ctypes.c_void_p),
                ("small_down_start", ctypes.c_void_p), ("small_down_end", ctypes.c_void_p),
                ("mfma_min_tokens", ctypes.c_int32), ("mfma_small_min_tokens", ctypes.c_int32)]


class RouteOptions(ctypes.Structure):
    """struct moe_route_options: the opt-in router variant (selection-only
    bias, normalised and scaled weights)"""
    _fields_ = [("bias_select_only", ctypes.c_int32), ("normalize", ctypes.c_int32),
                ("scale", ctypes.c_float), ("top_p", ctypes.c_float)]


class PoolDesc(ctypes.Structure):
    """struct moe_expert_pool"""
    _fields_ = [
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("wbits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("pool", ctypes.c_void_p),
        ("expert_bytes", ctypes.c_size_t),
        ("shared", ctypes.c_void_p),
        ("slot_of", ctypes.c_void_p),
        ("n_slots", ctypes.c_int32),
    ]


class LayerDesc(ctypes.Structure):
    """struct moe_layer_desc: one layer of a stack (pool, router, counters)"""
    _fields_ = [("pool", PoolDesc), ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p),
                ("counters", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m int4_routed_expert_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        P = ctypes.POINTER(PoolDesc)
        L.moe_route_topk.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.moe_union.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_route_union.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        RO = ctypes.POINTER(RouteOptions)
        L.moe_route_topk_ex.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp, RO]
        L.moe_route_union_ex.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp, RO]
        L.moe_expert_forward.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_forward_ex.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                            ctypes.POINTER(ForwardOptions)]
        L.moe_hit_count.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_layer_step.argtypes = [P, vp, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, sz, vp, ctypes.POINTER(ForwardOptions)]
        L.moe_layer_step_noalloc.argtypes = [P, vp, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, ctypes.POINTER(ForwardOptions)]
        L.moe_layer_step_workspace_size.argtypes = [P, i32, i32]
        LD = ctypes.POINTER(LayerDesc)
        L.moe_stack_forward.argtypes = [LD, i32, i32, i32, f32, vp, vp, vp, sz, vp]
        L.moe_stack_workspace_size.argtypes = [LD, i32, i32, i32]
        L.moe_residual_rmsnorm.argtypes = [vp, vp, vp, i32, i32, f32, vp]
        L.moe_route_workspace_size.argtypes = [i32, i32]
        L.moe_forward_workspace_size.argtypes = [P, i32, i32]
        L.moe_workspace_size.argtypes = [P, i32, i32]
        L.moe_block_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_pack_expert.argtypes = [vp, P, vp]
        L.moe_cache_create.argtypes = [i32, i32, sz, sz, vp, vp, vp, ctypes.POINTER(vp)]
        L.moe_cache_create.restype = i32
        L.moe_cache_destroy.argtypes = [vp]
        L.moe_cache_destroy.restype = None
        L.moe_cache_place.argtypes = [vp, vp, i32, vp, vp, vp]
        L.moe_cache_place.restype = i32
        L.moe_cache_forward.argtypes = [vp, P, vp, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                        sz, vp, vp, vp]
        L.moe_cache_forward.restype = i32
        L.moe_cache_stats.argtypes = [vp, vp, vp]
        L.moe_cache_stats.restype = i32
        for name in ("moe_cache_pin", "moe_cache_prefetch"):
            getattr(L, name).argtypes = [vp, vp, i32, vp, vp, vp]
            getattr(L, name).restype = i32
        L.moe_cache_resident.argtypes = [vp, vp, vp]
        L.moe_cache_resident.restype = i32
        L.moe_usage_write.argtypes = [ctypes.c_char_p, vp, i32, i32]
        L.moe_usage_write.restype = i32
        L.moe_usage_read.argtypes = [ctypes.c_char_p, vp, i32, i32]
        L.moe_usage_read.restype = i32
        L.moe_usage_hottest.argtypes = [vp, i32, i32, vp]
        L.moe_usage_hottest.restype = i32
        L.moe_strerror.argtypes = [i32]
        L.moe_strerror.restype = ctypes.c_char_p
        for name in ("moe_route_topk", "moe_route_topk_ex", "moe_union", "moe_route_union",
                     "moe_route_union_ex", "moe_expert_forward",
                     "moe_expert_forward_ex", "moe_hit_count", "moe_layer_step",
                     "moe_layer_step_noalloc", "moe_stack_forward",
                     "moe_residual_rmsnorm", "moe_pack_expert"):
            getattr(L, name).restype = i32
        for name in ("moe_route_workspace_size", "moe_forward_workspace_size",
                     "moe_workspace_size", "moe_layer_step_workspace_size", "moe_block_bytes",
                     "moe_stack_workspace_size"):
            getattr(L, name).restype = sz
        _lib = L
    return _lib


_probe_lib = None


def probe_lib():
    """The loaded libmoe_probe.so: measured ceilings of the GPU (a streaming
    read, a loop of matrix-core products), not part of the layer step."""
    global _probe_lib
    if _probe_lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                              "`python -m int4_routed_expert_gemv_amd.build`")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_probe_stream_read.argtypes = [vp, sz, i32, i32, vp, sz, vp, vp, vp]
        L.moe_probe_mfma_f16.argtypes = [vp, i32, i32, vp, vp, vp]
        for name in PROBE_EXPORTED:
            getattr(L, name).restype = i32
        _probe_lib = L
    return _probe_lib


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def _check(status: int, call: str):
    if status != MOE_OK:
        raise MoeError(status, call)


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")


# --------------------------------------------------------------------- sizes

def block_bytes(d_model, d_ff, wbits, group) -> int:
    return int(lib().moe_block_bytes(d_model, d_ff, wbits, group))


def route_workspace_size(n_tokens, n_experts) -> int:
    return int(lib().moe_route_workspace_size(n_tokens, n_experts))


def forward_workspace_size(pool: PoolDesc, n_tokens, k) -> int:
    return int(lib().moe_forward_workspace_size(ctypes.byref(pool), n_tokens, k))


def workspace_size(pool: PoolDesc, n_tokens, k) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(pool), n_tokens, k))


def layer_step_workspace_size(pool: PoolDesc, n_tokens, k) -> int:
    return int(lib().moe_layer_step_workspace_size(ctypes.byref(pool), n_tokens, k))


# --------------------------------------------------------------------- calls

def _route_opt(options):
    """None, or a RouteOptions pointer from a RouteOptions or a dict of its fields."""
    if options is None:
        return None
    if isinstance(options, dict):
        options = RouteOptions(int(options.get("bias_select_only", 0)),
                               int(options.get("normalize", 0)),
                               float(options.get("scale", 1.0)),
                               float(options.get("top_p", 0.0)))
    return ctypes.byref(options)


def route_topk(x, w_router, b_router, k, topk_ids, topk_w, workspace, stream=None, options=None):
    """moe_route_topk, or moe_route_topk_ex when options (RouteOptions or a
    dict with bias_select_only / normalize / scale) are given."""
    import torch
    _expect(x, torch.float32, "x")
    _expect(w_router, torch.float32, "w_router")
    _expect(b_router, torch.float32, "b_router")
    _expect(topk_ids, torch.int32, "topk_ids")
    _expect(topk_w, torch.float32, "topk_w")
    N, d = x.shape
    E = w_router.shape[0]
    args = (_ptr(x), N, d, _ptr(w_router), _ptr(b_router), E, k, _ptr(topk_ids), _ptr(topk_w),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if options is None:
        _check(lib().moe_route_topk(*args), "moe_route_topk")
    else:
        _check(lib().moe_route_topk_ex(*args, _route_opt(options)), "moe_route_topk_ex")


def union(topk_ids, n_experts, union_ids, n_union, expert_offsets, perm, stream=None):
    import torch
    for t, n in ((topk_ids, "topk_ids"), (union_ids, "union_ids"), (n_union, "n_union"),
                 (expert_offsets, "expert_offsets"), (perm, "perm")):
        _expect(t, torch.int32, n)
    N, k = topk_ids.shape
    _check(lib().moe_union(_ptr(topk_ids), N, k, n_experts, _ptr(union_ids), _ptr(n_union),
                           _ptr(expert_offsets), _ptr(perm), _stream(stream)), "moe_union")


def layer_step(pool: PoolDesc, x, w_router, b_router, k, topk_ids, topk_w, union_ids, n_union,
               expert_offsets, perm, counters, y, workspace, stream=None,
               options: ForwardOptions | None = None):
    """moe_layer_step: route_union then expert_forward in one call (one token:
    three launches, the routing inside the gate/up kernel); options as for
    expert_forward."""
    import torch
    _expect(x, torch.float32, "x")
    _expect(w_router, torch.float32, "w_router")
    _expect(b_router, torch.float32, "b_router")
    _expect(topk_w, torch.float32, "topk_w")
    _expect(y, torch.float32, "y")
    for t, n in ((topk_ids, "topk_ids"), (union_ids, "union_ids"), (n_union, "n_union"),
                 (expert_offsets, "expert_offsets"), (perm, "perm")):
        _expect(t, torch.int32, n)
    if counters is not None and counters.dtype not in (torch.int64, torch.uint64):
        raise TypeError("counters: expected a 64-bit integer tensor")
    if w_router.shape[0] != pool.n_experts:
        raise ValueError("w_router: expected one row per routed expert of the pool")
    N, d = x.shape
    _check(lib().moe_layer_step(ctypes.byref(pool), _ptr(x), N, d, _ptr(w_router), _ptr(b_router),
                                k, _ptr(topk_ids), _ptr(topk_w), _ptr(union_ids), _ptr(n_union),
                                _ptr(expert_offsets), _ptr(perm), _ptr(counters), _ptr(y),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream), None if options is None else ctypes.byref(options)),
           "moe_layer_step")


def layer_step_noalloc(pool: PoolDesc, x, w_router, b_router, k, topk_ids, topk_w, union_ids,
                       n_union, expert_offsets, perm, counters, y, stream=None,
                       options: ForwardOptions | None = None):
    """moe_layer_step_noalloc: layer_step with the library's own workspace
    array (no workspace argument, nothing allocated); raises MoeError with
    MOE_EWORKSPACE when the step needs more than MOE_SCRATCH_BYTES."""
    import torch
    _expect(x, torch.float32, "x")
    _expect(w_router, torch.float32, "w_router")
    _expect(b_router, torch.float32, "b_router")
    _expect(topk_w, torch.float32, "topk_w")
    _expect(y, torch.float32, "y")
    for t, n in ((topk_ids, "topk_ids"), (union_ids, "union_ids"), (n_union, "n_union"),
                 (expert_offsets, "expert_offsets"), (perm, "perm")):
        _expect(t, torch.int32, n)
    if counters is not None and counters.dtype not in (torch.int64, torch.uint64):
        raise TypeError("counters: expected a 64-bit integer tensor")
    if w_router.shape[0] != pool.n_experts:
        raise ValueError("w_router: expected one row per routed expert of the pool")
    N, d = x.shape
    _check(lib().moe_layer_step_noalloc(ctypes.byref(pool), _ptr(x), N, d, _ptr(w_router),
                                        _ptr(b_router), k, _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(union_ids), _ptr(n_union), _ptr(expert_offsets),
                                        _ptr(perm), _ptr(counters), _ptr(y), _stream(stream),
                                        None if options is None else ctypes.byref(options)),
           "moe_layer_step_noalloc")


def route_union(x, w_router, b_router, k, topk_ids, topk_w, union_ids, n_union, expert_offsets,
                perm, counters, workspace, stream=None, options=None):
    """moe_route_union: route_topk, union and (counters not None) hit_count in one call
    (moe_route_union_ex when options are given, as in route_topk)."""
    import torch
    _expect(x, torch.float32, "x")
    _expect(w_router, torch.float32, "w_router")
    _expect(b_router, torch.float32, "b_router")
    _expect(topk_w, torch.float32, "topk_w")
    for t, n in ((topk_ids, "topk_ids"), (union_ids, "union_ids"), (n_union, "n_union"),
                 (expert_offsets, "expert_offsets"), (perm, "perm")):
        _expect(t, torch.int32, n)
    if counters is not None and counters.dtype not in (torch.int64, torch.uint64):
        raise TypeError("counters: expected a 64-bit integer tensor")
    N, d = x.shape
    E = w_router.shape[0]
    args = (_ptr(x), N, d, _ptr(w_router), _ptr(b_router), E, k, _ptr(topk_ids), _ptr(topk_w),
            _ptr(union_ids), _ptr(n_union), _ptr(expert_offsets), _ptr(perm), _ptr(counters),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if options is None:
        _check(lib().moe_route_union(*args), "moe_route_union")
    else:
        _check(lib().moe_route_union_ex(*args, _route_opt(options)), "moe_route_union_ex")


def hit_count(topk_ids, n_experts, counters, stream=None):
    import torch
    _expect(topk_ids, torch.int32, "topk_ids")
    if counters.dtype not in (torch.int64, torch.uint64):
        raise TypeError("counters: expected a 64-bit integer tensor")
    N, k = topk_ids.shape
    _check(lib().moe_hit_count(_ptr(topk_ids), N, k, n_experts, _ptr(counters), _stream(stream)),
           "moe_hit_count")


def expert_forward(pool: PoolDesc, x, k, topk_w, union_ids, n_union, expert_offsets, perm, y,
                   workspace, stream=None, options: ForwardOptions | None = None):
    """moe_expert_forward, or moe_expert_forward_ex when options are given."""
    import torch
    _expect(x, torch.float32, "x")
    _expect(topk_w, torch.float32, "topk_w")
    _expect(y, torch.float32, "y")
    N = x.shape[0]
    args = (ctypes.byref(pool), _ptr(x), N, k, _ptr(topk_w), _ptr(union_ids), _ptr(n_union),
            _ptr(expert_offsets), _ptr(perm), _ptr(y), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if options is None:
        _check(lib().moe_expert_forward(*args), "moe_expert_forward")
    else:
        _check(lib().moe_expert_forward_ex(*args, ctypes.byref(options)), "moe_expert_forward_ex")


def layer_descs(layers):
    """A ctypes array of LayerDesc from (pool descriptor, w_router, b_router,
    counters) tuples (tensors or None)."""
    arr = (LayerDesc * len(layers))()
    for i, (desc, wr, b, cnt) in enumerate(layers):
        arr[i] = LayerDesc(desc, _ptr(wr), _ptr(b), _ptr(cnt))
    return arr


def stack_workspace_size(layers, n_tokens, k) -> int:
    """layers: the result of layer_descs()"""
    return int(lib().moe_stack_workspace_size(layers, len(layers), n_tokens, k))


def stack_forward(layers, h, k, workspace, topk_ids_out=None, eps=1e-6, stream=None):
    """moe_stack_forward: h [N][d] (in: the stack's input, out: its output)
    through every layer of `layers` (layer_descs()), chained by the residual
    RMS norm; topk_ids_out [L][N][k] int32 or None."""
    import torch
    _expect(h, torch.float32, "h")
    _expect(topk_ids_out, torch.int32, "topk_ids_out")
    N = h.shape[0]
    _check(lib().moe_stack_forward(layers, len(layers), N, k, eps, _ptr(h), _ptr(topk_ids_out),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "moe_stack_forward")


def residual_rmsnorm(h, y, a, eps=1e-6, stream=None):
    N, d = h.shape
    _check(lib().moe_residual_rmsnorm(_ptr(h), _ptr(y), _ptr(a), N, d, eps, _stream(stream)),
           "moe_residual_rmsnorm")


# --------------------------------------------------------------------- pools

def pack_expert(canonical: np.ndarray, shape: PoolDesc, out: np.ndarray | None = None) -> np.ndarray:
    """Canonical block (host bytes) -> device layout (host bytes); in place if out is canonical."""
    canonical = np.ascontiguousarray(canonical, np.uint8)
    out = canonical if out is None else out
    _check(lib().moe_pack_expert(canonical.ctypes.data, ctypes.byref(shape), out.ctypes.data),
           "moe_pack_expert")
    return out


class DevicePool:
    """One layer's experts resident in HBM: packed blocks plus the descriptor.

    blocks: uint8 [n_experts][stride] canonical blocks (host); packed in place.
    shared: uint8 [stride or block bytes] canonical shared-expert block, or None.
    """

    def __init__(self, d_model, d_ff, n_experts, wbits, group, blocks, shared, device="cuda"):
        import torch
        bb = block_bytes(d_model, d_ff, wbits, group)
        if bb == 0:
            raise MoeError(MOE_ESHAPE, "moe_block_bytes")
        stride = (bb + MOE_ALIGN - 1) // MOE_ALIGN * MOE_ALIGN
        self.desc = PoolDesc(d_model, d_ff, n_experts, wbits, group, None, stride, None)
        assert blocks.shape[0] == n_experts and blocks.shape[1] >= bb
        if blocks.shape[1] != stride:
            padded = np.zeros((n_experts, stride), np.uint8)
            padded[:, :blocks.shape[1]] = blocks
            blocks = padded
        for e in range(n_experts):
            pack_expert(blocks[e], self.desc)
        self.pool = torch.from_numpy(blocks).to(device)
        self.desc.pool = self.pool.data_ptr()
        self.shared = None
        if shared is not None:
            sh = np.zeros(stride, np.uint8)
            sh[:bb] = shared[:bb]
            pack_expert(sh, self.desc)
            self.shared = torch.from_numpy(sh).to(device)
            self.desc.shared = self.shared.data_ptr()
        if self.desc.pool % MOE_ALIGN or (self.shared is not None and self.desc.shared % MOE_ALIGN):
            raise MoeError(MOE_EALIGN, "DevicePool")
        self.stride = stride
        self.block_bytes = bb


class ExpertCache:
    """A layer's routed experts in pinned host memory with an HBM cache of
    n_slots block slots (moe_cache_*). host_blocks: pinned uint8 tensor
    [n_experts][stride] of device-layout blocks (pack_expert output)."""

    def __init__(self, pool_shape: PoolDesc, n_slots, host_blocks, device="cuda"):
        import torch
        E, stride = host_blocks.shape
        if E != pool_shape.n_experts or stride % MOE_ALIGN:
            raise ValueError("host_blocks must be [n_experts][stride], stride a multiple of 256")
        if not host_blocks.is_pinned():
            raise ValueError("host_blocks must be pinned host memory")
        bb = block_bytes(pool_shape.d_model, pool_shape.d_ff, pool_shape.wbits, pool_shape.group)
        self.host_blocks = host_blocks
        self.slots = torch.empty(n_slots * stride, dtype=torch.uint8, device=device)
        self.table = torch.empty(E, dtype=torch.int32, device=device)
        self.n_slots = n_slots
        h = ctypes.c_void_p()
        _check(lib().moe_cache_create(E, n_slots, bb, stride, host_blocks.data_ptr(),
                                      self.slots.data_ptr(), self.table.data_ptr(),
                                      ctypes.byref(h)), "moe_cache_create")
        self.handle = h
        self.desc = PoolDesc(pool_shape.d_model, pool_shape.d_ff, E, pool_shape.wbits,
                             pool_shape.group, self.slots.data_ptr(), stride, pool_shape.shared,
                             self.table.data_ptr(), n_slots)

    def place(self, union_ids_host, copy_stream=None, compute_stream=None) -> int:
        """Make the experts of union_ids_host (int32 numpy) resident; returns
        the number copied in."""
        ids = np.ascontiguousarray(union_ids_host, np.int32)
        missed = ctypes.c_int32(0)
        _check(lib().moe_cache_place(self.handle, ids.ctypes.data if ids.size else None, ids.size,
                                     _stream(copy_stream), _stream(compute_stream),
                                     ctypes.byref(missed)), "moe_cache_place")
        return int(missed.value)

    def forward(self, x, k, topk_w, union_ids, n_union, expert_offsets, perm, union_host, y,
                workspace, copy_stream=None, compute_stream=None) -> int:
        """moe_cache_forward: Place the union (union_host, int32 numpy) and
        run the expert math with the copies overlapping the resident experts'
        kernels; returns the number of experts copied in."""
        ids = np.ascontiguousarray(union_host, np.int32)
        missed = ctypes.c_int32(0)
        N = x.shape[0]
        _check(lib().moe_cache_forward(self.handle, ctypes.byref(self.desc), _ptr(x), N, k,
                                       _ptr(topk_w), _ptr(union_ids), _ptr(n_union),
                                       _ptr(expert_offsets), _ptr(perm),
                                       ids.ctypes.data if ids.size else None, ids.size, _ptr(y),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(copy_stream), _stream(compute_stream),
                                       ctypes.byref(missed)), "moe_cache_forward")
        return int(missed.value)

    def pin(self, ids_host, copy_stream=None, compute_stream=None) -> int:
        """Pin these experts (replacing the previous pin set); returns the
        number copied in."""
        ids = np.ascontiguousarray(ids_host, np.int32)
        missed = ctypes.c_int32(0)
        _check(lib().moe_cache_pin(self.handle, ids.ctypes.data if ids.size else None, ids.size,
                                   _stream(copy_stream), _stream(compute_stream),
                                   ctypes.byref(missed)), "moe_cache_pin")
        return int(missed.value)

    def prefetch(self, ids_host, copy_stream=None, compute_stream=None) -> int:
        """Start copying these experts in (a hint; the next place waits for
        the copies); returns the number of copies started."""
        ids = np.ascontiguousarray(ids_host, np.int32)
        n = ctypes.c_int32(0)
        _check(lib().moe_cache_prefetch(self.handle, ids.ctypes.data if ids.size else None,
                                        ids.size, _stream(copy_stream), _stream(compute_stream),
                                        ctypes.byref(n)), "moe_cache_prefetch")
        return int(n.value)

    def resident(self):
        """(slot_of[E], pinned[E]) on the host."""
        E = self.table.numel()
        so, pn = np.empty(E, np.int32), np.empty(E, np.int32)
        _check(lib().moe_cache_resident(self.handle, so.ctypes.data, pn.ctypes.data),
               "moe_cache_resident")
        return so, pn.astype(bool)

    def stats(self):
        h, m = ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(lib().moe_cache_stats(self.handle, ctypes.byref(h), ctypes.byref(m)), "moe_cache_stats")
        return int(h.value), int(m.value)

    def close(self):
        if getattr(self, "handle", None):
            lib().moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def usage_write(path, counters):
    """Save per-layer hit counters (uint64/int64 numpy [n_layers][n_experts])
    to a usage file (moe_usage_write)."""
    c = np.ascontiguousarray(np.atleast_2d(counters).astype(np.uint64))
    _check(lib().moe_usage_write(os.fsencode(path), c.ctypes.data, c.shape[0], c.shape[1]),
           "moe_usage_write")


def usage_read(path, n_layers, n_experts):
    """Load a usage file written by usage_write (moe_usage_read)."""
    c = np.zeros((n_layers, n_experts), np.uint64)
    _check(lib().moe_usage_read(os.fsencode(path), c.ctypes.data, n_layers, n_experts),
           "moe_usage_read")
    return c


def usage_hottest(counters_row, n):
    """The n experts with the most hits in one layer's counters, most first,
    ties to the lower id (moe_usage_hottest)."""
    c = np.ascontiguousarray(counters_row, np.uint64)
    ids = np.empty(n, np.int32)
    _check(lib().moe_usage_hottest(c.ctypes.data, c.size, n, ids.ctypes.data if n else None),
           "moe_usage_hottest")
    return ids
