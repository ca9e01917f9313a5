"""Seeded layer workloads for the parity tests, and the input-regeneration rule.

Routing is an integer decision taken on float32 scores. The GPU and the
oracle compute those scores with different rounding, so a token whose
adjacent top-(k+1) scores differ by less than 1e-6 could be ranked either way.
Such tokens are redrawn from the next attempt of their random stream until
every gap is clear (a test-data policy; the library itself always returns the
tie-broken ranking). The decision uses the oracle's scores only.
"""
import numpy as np

import oracle
import synth

GAP = 1e-6


def small_gap_tokens(scores: np.ndarray, k: int, gap: float = GAP) -> np.ndarray:
    """Indices of tokens with an adjacent gap < gap among their k+1 best scores."""
    E = scores.shape[1]
    m = min(k + 1, E)
    top = -np.sort(-scores.astype(np.float64), axis=1)[:, :m]
    if m < 2:
        return np.zeros(0, np.int64)
    return np.nonzero((top[:, :-1] - top[:, 1:] < gap).any(axis=1))[0]


def layer_inputs(cfg: synth.Config, layer: int = 0, max_attempts: int = 64):
    """x (with regenerated tokens), Wr, b, attempts per token, number redrawn."""
    wr, b = synth.router(cfg, layer)
    N, k = cfg.n_tokens, cfg.k
    attempts = np.zeros(N, np.int64)
    x = synth.tokens(cfg, attempts, layer)
    flagged = small_gap_tokens(oracle.router(x, wr, b), k)
    redrawn = set()
    while len(flagged):
        for t in flagged:
            attempts[t] += 1
            if attempts[t] > max_attempts:
                raise RuntimeError(f"token {t}: no clear top-{k} after {max_attempts} draws")
            redrawn.add(int(t))
        xs = synth.tokens(cfg, attempts, layer)
        x[flagged] = xs[flagged]
        sub = oracle.router(x[flagged], wr, b)
        flagged = flagged[small_gap_tokens(sub, k)]
    return x, wr, b, attempts, len(redrawn)


def canonical_pool(cfg: synth.Config, layer: int = 0):
    """(routed blocks uint8 [E][block_bytes], shared block uint8 [block_bytes])."""
    spec = cfg.layers[layer]
    blocks = synth.expert_pool(cfg, layer)
    shared = synth.shared_block(cfg, layer)
    return blocks, shared


def rel_err_rows(y, ref):
    """Per token: max_i |y - ref| / max_i |ref| (normwise relative error)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return num / np.maximum(den, 1e-30)


# ---------------------------------------------------------------- layer stacks

RMS_EPS = 1e-6


def stack_chain(cfg: synth.Config, attempts, tokens=None, on_layer=None):
    """Oracle pass through a stack of layers with residual chaining:
    h_0 = x, a_l = h_l / sqrt(mean(h_l^2) + eps), y_l = layer_l(a_l),
    h_{l+1} = h_l + y_l. Each layer's pool is drawn, used and dropped in turn.

    tokens: indices of the tokens to run (default: all). on_layer(l, spec,
    a_l, ref, blocks, shared, wr, b) is called after the oracle of layer l,
    with the canonical blocks still intact. Returns the indices (within
    `tokens`) of tokens with a top-(k+1) gap below GAP at some layer."""
    N = cfg.n_tokens
    tokens = np.arange(N) if tokens is None else np.asarray(tokens)
    x = synth.tokens(cfg, attempts)[tokens]
    h = x.astype(np.float64)
    flagged = set()
    for l, spec in enumerate(cfg.layers):
        a = oracle.rms_normalize(h, RMS_EPS)
        wr, b = synth.router(cfg, l)
        blocks, shared = canonical_pool(cfg, l)
        ref = oracle.layer_step(a, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits,
                                spec.group)
        flagged.update(small_gap_tokens(ref["scores"], cfg.k).tolist())
        if on_layer is not None:
            on_layer(l, spec, a, ref, blocks, shared, wr, b)
        del blocks
        h = h + ref["y"]
    return sorted(flagged)
