"""Seeded synthetic inputs for the routed-expert layer step.

This package draws numbers only: token activations, router weights and biases,
and canonical expert blocks. It holds none of the layer's arithmetic. The CPU
oracle and the GPU path both consume what it produces; neither imports the
other.

The workloads are GLM-5.2-shaped MoE layers (the Colibri pages describe
GLM-5.2 with 75 MoE layers of 256 experts, about 19 MB per int4 expert, a
shared expert per layer and an int8 draft head). No trained weights are
available, so every tensor is drawn from the distributions listed in
``CONFIGS``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED = 0
# stream tags (must match synth.c)
T_X, T_WR, T_BIAS = 1, 2, 3


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, vp, sz = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64] * 6
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_fill_bytes.argtypes = [u64, vp, sz]
        L.synth_fill_uniform.argtypes = [u64, vp, sz, ctypes.c_double, ctypes.c_double]
        L.synth_fill_normal.argtypes = [u64, vp, sz, ctypes.c_double, ctypes.c_double]
        L.synth_permutation.argtypes = [u64, vp, ctypes.c_int]
        L.synth_block_bytes.restype = sz
        L.synth_block_bytes.argtypes = [ctypes.c_int] * 4
        L.synth_expert_block.argtypes = [u64, u64, u64, u64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         ctypes.c_double, vp]
        L.synth_expert_pool.argtypes = [u64, u64, u64, u64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_double, vp, sz]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerSpec:
    """One MoE layer's shapes and draw distributions."""
    d: int                      # d_model
    f: int                      # d_ff of every expert (routed and shared)
    n_experts: int              # routed experts
    wbits: int                  # 4 (int4 nibbles) or 8 (int8)
    group: int                  # scale group along the input dim; 0 = one per row
    scale_lo: float
    scale_hi: float
    bias: str                   # "zero" or "zipf"
    zipf_s: float = 1.1
    router_std: float = 0.05


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    n_tokens: int
    k: int
    layers: tuple               # LayerSpec per layer, in order
    description: str = ""

    @property
    def layer(self) -> LayerSpec:
        return self.layers[0]


def _glm(bias, wbits=4, group=128, lo=0.002, hi=0.01):
    return LayerSpec(d=6144, f=2048, n_experts=256, wbits=wbits, group=group,
                     scale_lo=lo, scale_hi=hi, bias=bias)


CONFIGS = {
    "tiny": Config(
        "tiny", 1, n_tokens=4, k=1,
        layers=(LayerSpec(d=256, f=128, n_experts=16, wbits=4, group=32,
                          scale_lo=0.005, scale_hi=0.02, bias="zero"),),
        description="d_model=256, d_ff=128, 16 routed + 1 shared, top-1, 4 tokens"),
    "decode1": Config(
        "decode1", 2, n_tokens=1, k=1, layers=(_glm("zero"),),
        description="GLM-5.2-shaped decode layer: d=6144, d_ff=2048, 256+1 experts, top-1, 1 token"),
    "decode64": Config(
        "decode64", 3, n_tokens=64, k=8, layers=(_glm("zipf"),),
        description="batched decode: 64 tokens, top-8, Zipf(1.1) log-popularity router bias"),
    "prefill4096": Config(
        "prefill4096", 4, n_tokens=4096, k=8, layers=(_glm("zero"),),
        description="prefill: 4096 tokens, top-8, flat router bias"),
    "stack8_draft": Config(
        "stack8_draft", 5, n_tokens=256, k=8,
        layers=tuple([_glm("zipf")] * 8
                     + [_glm("zipf", wbits=8, group=0, lo=0.002 / 16, hi=0.01 / 16)]),
        description="8 int4 layers + int8 per-row-scale draft layer, 256 tokens, top-8, "
                    "Zipf(1.1) bias per layer, RMS-normalised residual chaining"),
}


def block_bytes(spec: LayerSpec) -> int:
    """Bytes of one canonical expert block."""
    return int(lib().synth_block_bytes(spec.d, spec.f, spec.wbits, spec.group))


def canonical_offsets(spec: LayerSpec) -> dict:
    """Byte offsets of the six arrays inside a canonical block."""
    d, f, wb, g = spec.d, spec.f, spec.wbits, spec.group
    q = d * f * wb // 8
    ns_gu = f * (d // g) if g else f
    ns_dn = d * (f // g) if g else d
    s0 = 3 * q
    return dict(gate_q=0, up_q=q, down_q=2 * q, gate_s=s0, up_s=s0 + 4 * ns_gu,
                down_s=s0 + 8 * ns_gu, q_bytes=q, ns_gu=ns_gu, ns_dn=ns_dn,
                total=s0 + 4 * (2 * ns_gu + ns_dn))


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------

def key(cfg_id, layer, tensor, index, attempt=0, seed=SEED) -> int:
    return int(lib().synth_key(seed, cfg_id, layer, tensor, index, attempt))


def normal(k: int, n: int, mean=0.0, std=1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_fill_normal(k, _ptr(out), n, mean, std)
    return out


def uniform(k: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_fill_uniform(k, _ptr(out), n, lo, hi)
    return out


def random_bytes(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().synth_fill_bytes(k, _ptr(out), n)
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, _ptr(out), n)
    return out


def tokens(cfg: Config, attempts=None, layer: int = 0) -> np.ndarray:
    """x[N][d] float32, token t drawn N(0,1) from stream (T_X, t, attempts[t])."""
    spec = cfg.layers[layer]
    N, d = cfg.n_tokens, spec.d
    attempts = np.zeros(N, np.int64) if attempts is None else np.asarray(attempts)
    x = np.empty((N, d), np.float32)
    for t in range(N):
        x[t] = normal(key(cfg.cfg_id, layer, T_X, t, int(attempts[t])), d)
    return x


def router(cfg: Config, layer: int = 0):
    """(Wr[E][d] float32 ~ N(0, router_std), b[E] float32)."""
    spec = cfg.layers[layer]
    E, d = spec.n_experts, spec.d
    wr = normal(key(cfg.cfg_id, layer, T_WR, 0), E * d, 0.0, spec.router_std).reshape(E, d)
    if spec.bias == "zero":
        b = np.zeros(E, np.float32)
    elif spec.bias == "zipf":
        # log-popularity: expert of popularity rank r (1 = hottest) gets -s*ln(r)
        rank = permutation(key(cfg.cfg_id, layer, T_BIAS, 0), E).astype(np.float64) + 1.0
        b = (-spec.zipf_s * np.log(rank)).astype(np.float32)
    else:
        raise ValueError(spec.bias)
    return wr, b


def expert_pool(cfg: Config, layer: int = 0, first: int = 0, count=None,
                stride=None, out: np.ndarray | None = None) -> np.ndarray:
    """Canonical blocks of experts first..first+count-1 as uint8[count][stride].
    Expert id n_experts is the shared expert."""
    spec = cfg.layers[layer]
    count = spec.n_experts - first if count is None else count
    bb = block_bytes(spec)
    stride = bb if stride is None else stride
    if out is None:
        out = np.zeros((count, stride), np.uint8)
    assert out.shape == (count, stride) and out.dtype == np.uint8
    lib().synth_expert_pool(SEED, cfg.cfg_id, layer, first, count, spec.d, spec.f,
                            spec.wbits, spec.group, spec.scale_lo, spec.scale_hi,
                            _ptr(out), stride)
    return out


def shared_block(cfg: Config, layer: int = 0) -> np.ndarray:
    spec = cfg.layers[layer]
    return expert_pool(cfg, layer, first=spec.n_experts, count=1)[0]
