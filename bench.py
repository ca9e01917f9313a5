#!/usr/bin/env python3
"""Throughput of the routed-expert layer step on one MI355X.

A step is one pass of the whole layer step over one batch, one
moe_layer_step call on one stream: route + top-k, union + permutation and hit
counters, then expert math + combine (for one token the routing runs inside
the gate/up GEMV launch). Inputs are synthetic and already resident in HBM.

Default workload ("decode1"): one GLM-5.2-shaped decode layer (d_model 6144,
d_ff 2048, 256 routed + 1 shared int4 experts with float32 scales per 128,
top-1, 1 token per step). Successive steps walk through --layers independently
drawn layer pools (each its own router and experts), as a decode pass walks
through a model's layers, so the 256 MB Infinity Cache cannot serve a
repeated working set.

Prints one JSON line. `roofline` is for the gate/up kernel of the pass
(GEMV, 32-token or 128-token matrix-core) whose launches take longest, timed
with HIP events that the kernel dispatches take on the library's stream, on
an evenly spread sample of about 64 timed steps (event-taking launches cost
the host tens of microseconds, so the other steps run without them).
`roofline.measured_ceiling` is what the simplest kernel of the same kind
reaches on this GPU (a plain streaming read of the same bytes per launch, or
a loop of independent matrix-core products), beside the published peak.
`cpu_baseline` is the CPU oracle timed on this host on a bounded sample of
the same workload.
"""
import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s and expert-weight HBM GB/s (% of 8 TB/s peak) on 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense float16 matrix-core peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--config", default="decode1")
    p.add_argument("--tokens", type=int, default=None,
                   help="tokens per step instead of the workload's (e.g. a speculative "
                        "verify batch of 1 + drafts through the stack)")
    p.add_argument("--k", type=int, default=None, help="experts per token instead of the workload's")
    p.add_argument("--small-min", type=int, default=None,
                   help="experts with at least this many tokens take the 32-token matrix-core "
                        "pass (moe_forward_options.mfma_small_min_tokens; default: the library's)")
    p.add_argument("--group", type=int, default=None,
                   help="scale group of the int4 layers instead of the workload's (e.g. 64)")
    p.add_argument("--layers", type=int, default=8, help="layer pools rotated over the steps")
    p.add_argument("--batches", type=int, default=16, help="distinct token batches rotated")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run one plain device copy of 1 GiB (to scale HBM counters)")
    p.add_argument("--cache-stack", type=int, default=None, metavar="SLOTS",
                   help="decode through the int4 layers of the stack workload, each layer's "
                        "experts in pinned host memory with an HBM cache of SLOTS slots; "
                        "compares LRU, LRU + learned pins, LRU + lookahead prefetch, and both")
    p.add_argument("--stack-tokens", type=int, default=1, help="tokens per step for --cache-stack")
    p.add_argument("--pin", type=int, default=32, help="experts pinned per layer (--cache-stack)")
    p.add_argument("--lookahead-top", type=int, default=None,
                   help="--cache-stack: prefetch only each token's first M predicted experts")
    p.add_argument("--cache-slots", default=None,
                   help="comma-separated HBM slot counts: measure the Place stage (experts in "
                        "pinned host memory, an HBM cache of that many slots per layer) instead")
    return p.parse_args()


def copy_calibration():
    """One plain device-to-device copy kernel of exactly 1 GiB read + 1 GiB
    written, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n}), flush=True)


def kernel_source_hash():
    """Hash of the expert kernel sources with comments and blank space taken
    out (counters taken with other kernel code do not apply)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in ("expert_gemv.hip", "expert_mfma.hip", "internal.h"):
        with open(os.path.join(ROOT, "int4_routed_expert_gemv_amd", "csrc", name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config, kernel):
    """HBM bytes per launch of `kernel` on `config` from the committed counter
    summary, or None when there is none or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    entry = data.get(config, {}).get(kernel)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


class Hip:
    """HIP events through the runtime library (the kernels' own stream is torch's)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            # an event that no launch took: clear the runtime's last error so
            # that later checks (torch's included) do not report it
            self.L.hipGetLastError()
            raise AssertionError("event not recorded")
        return ms.value


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.cache_slots:
        cache_bench(args)
        return
    if args.cache_stack:
        cache_stack_bench(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.CONFIGS[args.config]
    if args.group is not None:
        base = dataclasses.replace(base, layers=tuple(
            dataclasses.replace(ls, group=args.group) if ls.wbits == 4 else ls
            for ls in base.layers))
    if args.tokens is not None:
        base = dataclasses.replace(base, n_tokens=args.tokens)
    if args.k is not None:
        base = dataclasses.replace(base, k=args.k)
    spec = base.layer
    stack = len(base.layers) > 1
    if stack:
        # a step is one pass through the whole stack (layers chained on the GPU)
        cfg = base
        L_rot = len(cfg.layers)
    else:
        L_rot = args.layers
        cfg = dataclasses.replace(base, layers=(spec,) * L_rot)
    N, k, E, d, f = cfg.n_tokens, cfg.k, spec.n_experts, spec.d, spec.f
    A = N * k
    nb = max(1, min(args.batches, args.steps + args.warmup))
    t_setup = time.time()

    # --- inputs resident in HBM -------------------------------------------
    pools, routers = [], []
    for l in range(L_rot):
        ls = cfg.layers[l]
        blocks = synth.expert_pool(cfg, l)
        shared = synth.shared_block(cfg, l)
        pools.append(moe.DevicePool(d, f, E, ls.wbits, ls.group, blocks, shared, dev))
        del blocks
        wr, b = synth.router(cfg, l)
        routers.append((torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)))
        print(f"[bench] layer pool {l + 1}/{L_rot} resident", file=sys.stderr, flush=True)
    tok_cfg = dataclasses.replace(cfg, n_tokens=N * nb)
    xs = torch.from_numpy(synth.tokens(tok_cfg).reshape(nb, N, d)).to(dev)
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    union_ids = torch.empty(E, dtype=torch.int32, device=dev)
    n_union = torch.empty(1, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(A, dtype=torch.int32, device=dev)
    counters = torch.zeros((L_rot, E), dtype=torch.int64, device=dev)
    y = torch.empty((N, d), dtype=torch.float32, device=dev)
    ws_bytes = max(moe.layer_step_workspace_size(p.desc, N, k) for p in pools)
    hbuf = torch.empty((N, d), dtype=torch.float32, device=dev)   # residual stream
    abuf = torch.empty((N, d), dtype=torch.float32, device=dev)   # normalised layer input
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # --- raw C-ABI calls with their arguments converted once ---------------
    Lb = moe.lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    hip = Hip()

    def step_args(s):
        l, bi = s % L_rot, s % nb
        x = abuf if stack else xs[bi]
        wr, b = routers[l]
        # Route, Union, Learn and the experts in one call (moe_layer_step)
        return (ctypes.byref(pools[l].desc), vp(x.data_ptr()), N, d, vp(wr.data_ptr()),
                vp(b.data_ptr()), k, vp(ids.data_ptr()), vp(w.data_ptr()),
                vp(union_ids.data_ptr()), vp(n_union.data_ptr()), vp(offsets.data_ptr()),
                vp(perm.data_ptr()), vp(counters[l].data_ptr()), vp(y.data_ptr()),
                vp(ws.data_ptr()), ws_bytes, stream)

    plans = [step_args(s) for s in range(L_rot if stack else L_rot * nb)]
    n_plan = len(plans)
    hip_rt = ctypes.CDLL("libamdhip64.so")
    hip_rt.hipMemcpyAsync.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]

    base_opts = None
    if args.small_min is not None:
        base_opts = moe.ForwardOptions()
        base_opts.mfma_small_min_tokens = args.small_min

    def run_layer(s, ev=None):
        opt = ev if ev is not None else base_opts
        rc = Lb.moe_layer_step(*plans[s % n_plan], None if opt is None else ctypes.byref(opt))
        if rc:
            raise RuntimeError(f"layer step failed with status {rc}")

    def run(s, ev=None):
        if not stack:
            run_layer(s, ev)
            return
        # h = x (device copy), then per layer: h += y (from layer 1 on),
        # a = rms(h), layer(a) -> y
        x = xs[s % nb]
        rc = hip_rt.hipMemcpyAsync(vp(hbuf.data_ptr()), vp(x.data_ptr()), x.numel() * 4, 3, stream)
        for l in range(L_rot):
            rc |= Lb.moe_residual_rmsnorm(vp(hbuf.data_ptr()), vp(y.data_ptr()) if l else None,
                                          vp(abuf.data_ptr()), N, d, ctypes.c_float(1e-6), stream)
            if rc:
                raise RuntimeError(f"stack step failed with status {rc}")
            run_layer(l, ev if l == 0 else None)

    # which experts each (layer, batch) step streams and on which kernels
    # (the library's default thresholds): experts with at least MFMA_MIN
    # tokens go to the 128-token matrix-core pass, those with at least
    # SMALL_MIN to the 32-token pass, the rest to the GEMVs; the shared
    # expert by the batch size
    MFMA_MIN = 32
    SMALL_MIN = args.small_min if args.small_min is not None else 2
    mfma_ok = spec.wbits == 4 and d % 64 == 0 and f % 64 == 0
    calib = {}

    MIN_BIG_ITEMS = 32  # fewer 128-token items than this join the 32-token pass
    GEMV_BATCH = 2      # batches of at most this many tokens keep every expert on the GEMV

    def pass_of(T):
        T = np.asarray(T)
        big = (T >= MFMA_MIN) & mfma_ok
        # batches of up to GEMV_BATCH tokens stay on the GEMV (the library's default)
        small = ~big & (T >= SMALL_MIN) & mfma_ok & (N > GEMV_BATCH or args.small_min is not None)
        if big.any() and np.sum((T[big] + 127) // 128) < MIN_BIG_ITEMS:
            small, big = small | big, np.zeros_like(big)
        return np.where(big, 1, np.where(small, 2, 0))

    def record(key, l):
        torch.cuda.synchronize()
        nu = int(n_union.item())
        uid = union_ids[:nu].cpu().numpy()
        off = offsets.cpu().numpy()
        T = np.concatenate([off[uid + 1] - off[uid], [N]])  # routed, then shared
        ps = pass_of(T)
        c = dict(union=nu, wbits=cfg.layers[l].wbits, group=cfg.layers[l].group)
        for name, code in (("gemv", 0), ("mfma", 1), ("small", 2)):
            c[name + "_experts"] = int((ps == code).sum())
            c[name + "_tokens"] = int(T[ps == code].sum())
        # a 128-token group's remainder of at most 32 tokens past a full item
        # runs on the 32-token pass (its weights streamed there once more)
        if mfma_ok and (N > GEMV_BATCH or args.small_min is not None) and SMALL_MIN > 0:
            r = T % 128
            rem = (ps == 1) & (T > 128) & (r > 0) & (r <= 32)
            c["mfma_tokens"] -= int(r[rem].sum())
            c["small_tokens"] += int(r[rem].sum())
            c["small_experts"] += int(rem.sum())
        calib[key] = c

    if stack:
        x0 = xs[0]
        hip_rt.hipMemcpyAsync(vp(hbuf.data_ptr()), vp(x0.data_ptr()), x0.numel() * 4, 3, stream)
        for l in range(L_rot):
            Lb.moe_residual_rmsnorm(vp(hbuf.data_ptr()), vp(y.data_ptr()) if l else None,
                                    vp(abuf.data_ptr()), N, d, ctypes.c_float(1e-6), stream)
            run_layer(l)
            record(l, l)
    else:
        for s_ in range(n_plan):
            run(s_)
            record(s_, s_ % L_rot)
    for _ in range(args.warmup):
        run(_)
    torch.cuda.synchronize()
    mean_union = float(np.mean([c["union"] for c in calib.values()]))
    print(f"[bench] setup {time.time() - t_setup:.1f}s; mean union {mean_union:.1f}",
          file=sys.stderr, flush=True)

    # --- timed region -------------------------------------------------------
    K = args.steps
    # Kernel durations come from HIP events that the dispatches themselves
    # take (start and end of each expert kernel) on a sample of the timed
    # steps, evenly spread: about 64 of them, or every step of a short run.
    # Event-taking launches cost the host tens of microseconds per step, so
    # the other steps run without them.
    every = max(1, K // 64)
    sampled = [s_ for s_ in range(K) if s_ % every == 0]
    evs = {s_: moe.ForwardOptions(*[hip.event() for _ in range(12)], 0,
                                  args.small_min if args.small_min is not None else 0)
           for s_ in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(K):
        run(args.warmup + s_, evs.get(s_))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    def ms(e, a, b):
        try:
            return hip.elapsed_ms(getattr(e, a), getattr(e, b))
        except AssertionError:  # the kernel was not launched in that step
            return None

    # per pass: event-timed gate/up and down launches of every timed step
    timed = {}
    for name, pre in (("gemv", ""), ("mfma", "mfma_"), ("small", "small_")):
        timed[name] = ([ms(evs[s_], pre + "gateup_start", pre + "gateup_end") for s_ in sampled],
                       [ms(evs[s_], pre + "down_start", pre + "down_end") for s_ in sampled])
    for e in evs.values():
        for fld, _ in moe.ForwardOptions._fields_[:12]:
            hip.L.hipEventDestroy(getattr(e, fld))

    # --- algorithmic bytes and flops ------------------------------------------
    def sizes(c):
        bb = moe.block_bytes(d, f, c["wbits"], c["group"])
        q_gu = f * d * c["wbits"] // 8
        s_gu = f * (d // c["group"] if c["group"] else 1) * 4
        return bb, 2 * (q_gu + s_gu)

    # the calibration entry of the (first) layer the events of a step cover
    step_key = [0 if stack else (args.warmup + s_) % n_plan for s_ in range(K)]
    layer_keys = list(range(L_rot)) if stack else None
    expert_bytes = 0
    router_bytes = 0
    for s_ in range(K):
        keys = layer_keys if stack else [step_key[s_]]
        for key in keys:
            c = calib[key]
            bb, _ = sizes(c)
            expert_bytes += (c["union"] + 1) * bb
            router_bytes += E * d * 4 + E * 4
    ms_per_step = elapsed / K * 1e3
    tokens_per_s = N * K / elapsed
    expert_gbs = expert_bytes / 1e9 / elapsed

    def avg(v):
        v = [x for x in v if x is not None]
        return float(np.mean(v)) if v else None

    # Gate/up kernels of the three passes. The GEMV and 32-token passes are
    # HBM-bound: algorithmic bytes = gate and up codes + scales of every
    # expert the pass handles, once. The 128-token pass is matrix-core bound:
    # algorithmic flops = 2 (gate, up) x 2 x d x f per token it handles.
    steps_c = [calib[step_key[s_]] for s_ in sampled]  # the steps whose kernels were timed
    passes = {}
    for name in ("gemv", "small", "mfma"):
        gu_t, dn_t = timed[name]
        if not avg(gu_t):
            continue
        t_gu, t_dn = avg(gu_t) / 1e3, (avg(dn_t) / 1e3 if avg(dn_t) else None)
        gu_b = float(np.mean([c[name + "_experts"] * sizes(c)[1] for c in steps_c]))
        dn_b = float(np.mean([c[name + "_experts"] * (sizes(c)[0] - sizes(c)[1]) for c in steps_c]))
        fl = float(np.mean([4.0 * d * f * c[name + "_tokens"] for c in steps_c]))
        passes[name] = {"avg_launch_us": t_gu * 1e6, "bytes_per_launch": gu_b,
                        "achieved_GBps": gu_b / 1e9 / t_gu, "flops_per_launch": fl,
                        "achieved_TFLOPs": fl / 1e12 / t_gu,
                        "down_avg_launch_us": t_dn * 1e6 if t_dn else None,
                        "down_GBps": dn_b / 1e9 / t_dn if t_dn else None}
    labels = {"gemv": ("gemv_kernel<gate/up> (expert gate and up projections, SiLU product)",
                       "moe::gemv_kernel<true, 4, 1"),
              "small": ("mfma_kernel<gate/up, 32 tokens> (small-group gate and up on the "
                        "matrix cores)", "moe::mfma_kernel<true, 4, 2"),
              "mfma": ("mfma_kernel<gate/up, 128 tokens> (grouped GEMM of gate and up, SiLU "
                       "product)", "moe::mfma_kernel<true, 4, 8")}
    roof = None
    if passes:
        # the roofline is reported for the pass whose gate/up launch is longest
        top = max(passes, key=lambda n: passes[n]["avg_launch_us"])
        pz = passes[top]
        if top == "mfma":
            roof = {"bound": "mfma", "achieved": pz["achieved_TFLOPs"],
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": pz["achieved_TFLOPs"] / MFMA_F16_PEAK_TFLOPS}
        else:
            roof = {"bound": "hbm", "achieved": pz["achieved_GBps"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": pz["achieved_GBps"] / HBM_PEAK_GBS}
        roof["traffic"] = (None if args.tokens is not None or args.k is not None else measured_traffic(
            args.config if args.group is None else f"{args.config}_g{args.group}",
            labels[top][1]))
        roof["kernel"] = labels[top][0]
        roof["passes"] = passes
        roof["measured_ceiling"] = measured_ceiling(moe, hip, torch, roof["bound"],
                                                    pz["bytes_per_launch"], roof["achieved"])

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xf16->f32" if spec.wbits == 4 else "int8xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {base.description}" +
                         ("" if stack else f"; {L_rot} layer pools rotated") +
                         (f"; int4 scale groups of {args.group}" if args.group else "") +
                         (f"; {N} tokens per step" if args.tokens is not None else "") +
                         (f"; top-{k}" if args.k is not None else "")),
            "n_tokens": N, "k": k, "d_model": d, "d_ff": f, "n_experts": E,
            "wbits": spec.wbits, "group": spec.group, "layers_per_step": L_rot if stack else 1,
            "layer_pools": L_rot, "mean_union": mean_union,
        },
        "expert_GBps": expert_gbs,
        "expert_frac_of_peak": expert_gbs / HBM_PEAK_GBS,
        "step_GBps": (expert_bytes + router_bytes) / 1e9 / elapsed,
        "roofline": roof,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, spec, args, xs.cpu().numpy())
    print(json.dumps(result), flush=True)


def cache_bench(args):
    """Place stage: each layer's routed experts in pinned host memory, an HBM
    cache of C slots per layer (moe_cache_*, least recently used
    replacement). A step routes the batch (moe_route_union), copies the union
    to the host, places it (missing blocks copied on a second stream), then
    runs the expert math through the slot table. Reported per slot count:
    tokens/s, the hit rate over the timed steps and the bytes copied per
    token next to the L*k*S*(1-h) estimate (here L = 1 layer per step)."""
    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    dev = torch.device("cuda:0")
    base = synth.CONFIGS[args.config]
    if len(base.layers) > 1:
        sys.exit("--cache-slots measures single-layer workloads")
    spec = base.layer
    L_rot = max(1, min(args.layers, 4))
    cfg = dataclasses.replace(base, layers=(spec,) * L_rot)
    N, k, E, d, f = cfg.n_tokens, cfg.k, spec.n_experts, spec.d, spec.f
    nb = max(1, args.batches)  # distinct token batches cycled through (the access stream)
    layers = []
    for l in range(L_rot):
        pool = moe.DevicePool(d, f, E, spec.wbits, spec.group, synth.expert_pool(cfg, l),
                              synth.shared_block(cfg, l), dev)
        host = torch.empty((E, pool.stride), dtype=torch.uint8, pin_memory=True)
        host.copy_(pool.pool.view(E, pool.stride))
        shared = pool.shared
        desc = pool.desc
        del pool
        wr, b = synth.router(cfg, l)
        layers.append(dict(host=host, shared=shared, desc=desc, wr=torch.from_numpy(wr).to(dev),
                           b=torch.from_numpy(b).to(dev)))
        torch.cuda.empty_cache()
        print(f"[cache bench] layer {l + 1}/{L_rot} in pinned host memory", file=sys.stderr,
              flush=True)
    tok_cfg = dataclasses.replace(cfg, n_tokens=N * nb)
    xs = torch.from_numpy(synth.tokens(tok_cfg).reshape(nb, N, d)).to(dev)
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    uid = torch.empty(E, dtype=torch.int32, device=dev)
    nu = torch.empty(1, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(N * k, dtype=torch.int32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int64, device=dev)
    y = torch.empty((N, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.workspace_size(ly["desc"], N, k) for ly in layers), dtype=torch.uint8,
                     device=dev)
    copy_stream = torch.cuda.Stream()  # default priority
    block = moe.block_bytes(d, f, spec.wbits, spec.group)
    points = []
    for C in [int(c) for c in args.cache_slots.split(",")]:
        caches = [moe.ExpertCache(ly["desc"], C, ly["host"], dev) for ly in layers]

        def run(s_):
            ly, cache = layers[s_ % L_rot], caches[s_ % L_rot]
            x = xs[s_ % nb]
            moe.route_union(x, ly["wr"], ly["b"], k, ids, w, uid, nu, off, perm, cnt, ws)
            n = int(nu.item())
            cache.place(uid[:n].cpu().numpy(), copy_stream=copy_stream)
            moe.expert_forward(cache.desc, x, k, w, uid, nu, off, perm, y, ws)

        for s_ in range(args.warmup):
            run(s_)
        torch.cuda.synchronize()
        h0 = [c.stats() for c in caches]
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            run(args.warmup + s_)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        hits = sum(c.stats()[0] - h[0] for c, h in zip(caches, h0))
        misses = sum(c.stats()[1] - h[1] for c, h in zip(caches, h0))
        hr = hits / max(1, hits + misses)
        tok = N * args.steps
        points.append({"slots": C, "tokens_per_s": tok / el, "ms_per_step": el / args.steps * 1e3,
                       "hit_rate": hr, "misses_per_step": misses / args.steps,
                       "copied_bytes_per_token": misses * block / tok,
                       "estimate_bytes_per_token": k * block * (1 - hr),
                       "copied_GBps": misses * block / el / 1e9})
        print(f"[cache bench] {C} slots: {points[-1]}", file=sys.stderr, flush=True)
        for c in caches:
            c.close()
        del caches
    print(json.dumps({"metric": "layer-step tokens/s with experts placed from pinned host memory "
                                "into an HBM cache (Place stage)",
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic",
                      "config": {"workload": f"{cfg.name}: {base.description}; {L_rot} layers, "
                                             f"one cache per layer", "n_tokens": N, "k": k,
                                 "n_experts": E, "block_bytes": block},
                      "points": points}), flush=True)


def cache_stack_bench(args):
    """Place with the pages' two placement aids, on a decode stack: the int4
    layers of the stack workload (--layers of them) chained through the
    residual RMS norm, every layer's experts in pinned host memory with an
    HBM cache of SLOTS slots (moe_cache_*). Four policies, each on fresh
    caches over the same token stream:
      lru        Place only (least recently used replacement);
      pin        + the --pin hottest experts of each layer pinned, chosen from
                 the hit counters of a learning pass (moe_usage_hottest);
      lookahead  + while layer l computes, layer l+1's router runs on layer
                 l's normalised hidden state and its predicted union (each
                 token's first --lookahead-top ranked experts, all k by
                 default) is prefetched (moe_cache_prefetch), the copies
                 overlapping layer l's expert math;
      both       pins and lookahead.
    Reported per policy: tokens/s, the Place hit rate, bytes copied per token
    (prefetches included) and the lookahead's accuracy (the share of each
    layer's union that was predicted)."""
    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    dev = torch.device("cuda:0")
    base = synth.CONFIGS["stack8_draft"]
    int4 = [ls for ls in base.layers if ls.wbits == 4]
    L = max(2, min(args.layers, len(int4)))
    N = args.stack_tokens
    cfg = dataclasses.replace(base, layers=tuple(int4[:L]), n_tokens=N)
    k, C = cfg.k, args.cache_stack
    n_pin = min(args.pin, C - N * k)   # a union's unpinned experts always find slots
    if n_pin < 0:
        sys.exit(f"--cache-stack needs at least {N * k} slots for {N} token(s) of top-{k}")
    spec = cfg.layers[0]
    E, d, f = spec.n_experts, spec.d, spec.f
    layers = []
    for l in range(L):
        ls = cfg.layers[l]
        pool = moe.DevicePool(d, f, E, ls.wbits, ls.group, synth.expert_pool(cfg, l),
                              synth.shared_block(cfg, l), dev)
        host = torch.empty((E, pool.stride), dtype=torch.uint8, pin_memory=True)
        host.copy_(pool.pool.view(E, pool.stride))
        shared, desc = pool.shared, pool.desc
        del pool
        wr, b = synth.router(cfg, l)
        layers.append(dict(host=host, shared=shared, desc=desc, wr=torch.from_numpy(wr).to(dev),
                           b=torch.from_numpy(b).to(dev)))
        torch.cuda.empty_cache()
        print(f"[cache stack] layer {l + 1}/{L} in pinned host memory", file=sys.stderr, flush=True)
    nb = args.warmup + args.steps
    xs = torch.from_numpy(synth.tokens(dataclasses.replace(cfg, n_tokens=N * nb))
                          .reshape(nb, N, d)).to(dev)
    ids = torch.empty((N, k), dtype=torch.int32, device=dev)
    w = torch.empty((N, k), dtype=torch.float32, device=dev)
    pid = torch.empty((N, k), dtype=torch.int32, device=dev)
    pw = torch.empty((N, k), dtype=torch.float32, device=dev)
    uid = torch.empty(E, dtype=torch.int32, device=dev)
    nu = torch.empty(1, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(N * k, dtype=torch.int32, device=dev)
    y = torch.empty((N, d), dtype=torch.float32, device=dev)
    h = torch.empty((N, d), dtype=torch.float32, device=dev)
    a = torch.empty((N, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.workspace_size(ly["desc"], N, k) for ly in layers), dtype=torch.uint8,
                     device=dev)
    copy_stream = torch.cuda.Stream()  # default priority
    block = moe.block_bytes(d, f, spec.wbits, spec.group)
    Lb = moe.lib()

    def rmsnorm(first):
        rc = Lb.moe_residual_rmsnorm(h.data_ptr(), None if first else y.data_ptr(), a.data_ptr(),
                                     N, d, ctypes.c_float(1e-6), None)
        if rc:
            raise RuntimeError(f"moe_residual_rmsnorm failed with status {rc}")

    def token_step(s_, caches, cnt, lookahead, acc):
        h.copy_(xs[s_])
        copies = 0
        for l in range(L):
            ly, cache = layers[l], caches[l]
            rmsnorm(l == 0)
            moe.route_union(a, ly["wr"], ly["b"], k, ids, w, uid, nu, off, perm, cnt[l], ws)
            union = uid[:int(nu.item())].cpu().numpy()
            if acc is not None and l > 0 and acc["pred"] is not None:
                acc["hit"] += len(set(union.tolist()) & acc["pred"])
                acc["total"] += len(union)
            copies += cache.place(union, copy_stream=copy_stream)
            if lookahead and l + 1 < L:
                nxt = layers[l + 1]
                moe.route_topk(a, nxt["wr"], nxt["b"], k, pid, pw, ws)
                pred_ids = pid.cpu().numpy()
                pred = np.unique(pred_ids[:, :top] if top else pred_ids)
                if acc is not None:
                    acc["pred"] = set(pred.tolist())
                copies += caches[l + 1].prefetch(pred, copy_stream=copy_stream)
            moe.expert_forward(cache.desc, a, k, w, uid, nu, off, perm, y, ws)
        return copies

    learn_steps = max(1, args.warmup)
    top = args.lookahead_top   # ranked predictions kept per token (None: all k)
    points = []
    for policy in ("lru", "pin", "lookahead", "both"):
        caches = [moe.ExpertCache(ly["desc"], C, ly["host"], dev) for ly in layers]
        cnt = torch.zeros((L, E), dtype=torch.int64, device=dev)
        pinning = policy in ("pin", "both")
        lookahead = policy in ("lookahead", "both")
        for s_ in range(learn_steps):   # learning pass: fills the caches and the counters
            token_step(s_, caches, cnt, lookahead, None)
        torch.cuda.synchronize()
        if pinning:
            counters = cnt.cpu().numpy().astype(np.uint64)
            for l in range(L):
                caches[l].pin(moe.usage_hottest(counters[l], n_pin), copy_stream=copy_stream)
        torch.cuda.synchronize()
        st0 = [c.stats() for c in caches]
        acc = dict(hit=0, total=0, pred=None)
        copies = 0
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            acc["pred"] = None
            copies += token_step(learn_steps + s_, caches, cnt, lookahead, acc)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        hits = sum(c.stats()[0] - s0[0] for c, s0 in zip(caches, st0))
        misses = sum(c.stats()[1] - s0[1] for c, s0 in zip(caches, st0))
        tok = N * args.steps
        pt = {"policy": policy, "tokens_per_s": tok / el, "ms_per_token_step": el / args.steps * 1e3,
              "place_hit_rate": hits / max(1, hits + misses),
              "copied_bytes_per_token": copies * block / tok,
              "lookahead_accuracy": (acc["hit"] / acc["total"]) if lookahead and acc["total"]
              else None}
        points.append(pt)
        print(f"[cache stack] {pt}", file=sys.stderr, flush=True)
        for c in caches:
            c.close()
        del caches
    print(json.dumps({"metric": "decode tokens/s through a layer stack with experts placed from "
                                "pinned host memory into per-layer HBM caches (Place, learned "
                                "pinning, lookahead prefetch)",
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                      "learning_steps": learn_steps, "data": "synthetic",
                      "config": {"workload": f"{L} int4 layers of {cfg.name} chained, "
                                             f"{N} token(s) per step, top-{k}, Zipf(1.1) router "
                                             f"bias per layer", "slots_per_layer": C,
                                 "pinned_per_layer": n_pin, "lookahead_top": top or k,
                                 "n_experts": E,
                                 "block_bytes": block},
                      "points": points}), flush=True)


def measured_ceiling(moe, hip, torch, bound, bytes_per_launch, achieved):
    """What this GPU delivers to the simplest kernel of the same kind, beside
    the published peak: for an HBM-bound kernel, a plain streaming read of the
    same bytes per launch (moe_probe_stream_read, best of three wave shapes,
    buffers rotated past the 256 MB Infinity Cache); for the matrix-core pass,
    a loop of independent float16 MFMA products (moe_probe_mfma_f16). Timed
    with HIP events taken by the probe launches themselves."""
    import numpy as np
    L = moe.probe_lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    ev = [hip.event() for _ in range(2)]
    if bound == "hbm":
        nbytes = int(bytes_per_launch) // 1024 * 1024
        if nbytes < 1024:
            return None
        n_buf = max(2, -(-(1 << 30) // nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(n_buf)]
        sink = torch.empty(nbytes // 1024 + 1, dtype=torch.int32, device="cuda")
        best = None
        for ub, nw in ((3, 4), (6, 4), (12, 8)):
            ts = []
            for i in range(23):
                rc = L.moe_probe_stream_read(vp(bufs[i % n_buf].data_ptr()), nbytes, ub, nw,
                                             vp(sink.data_ptr()), sink.numel(), vp(ev[0]), vp(ev[1]),
                                             stream)
                assert rc == 0, rc
                torch.cuda.synchronize()
                if i >= 3:
                    ts.append(hip.elapsed_ms(ev[0], ev[1]))
            us = float(np.mean(ts)) * 1e3
            if best is None or us < best[0]:
                best = (us, ub, nw)
        del bufs
        value = nbytes / 1e9 / (best[0] * 1e-6)
        out = {"what": f"plain streaming read of {nbytes} B per launch, {best[1]} KB per wave, "
                       f"{best[2]}-wave workgroups ({best[0]:.2f} us)",
               "value": value, "unit": "GB/s", "frac": achieved / value}
    else:
        wgs, iters = 2048, 1000
        o = torch.empty(4 * wgs, dtype=torch.float32, device="cuda")
        ts = []
        for i in range(13):
            assert L.moe_probe_mfma_f16(vp(o.data_ptr()), wgs, iters, vp(ev[0]), vp(ev[1]), stream) == 0
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(hip.elapsed_ms(ev[0], ev[1]))
        sec = float(np.mean(ts)) * 1e-3
        value = wgs * 4 * iters * 4 * 16384 / sec / 1e12
        out = {"what": f"loop of independent v_mfma_f32_16x16x32_f16 on register operands, "
                       f"{wgs} workgroups of 4 waves",
               "value": value, "unit": "TFLOP/s", "frac": achieved / value}
    for e in ev:
        hip.L.hipEventDestroy(e)
    return out


def cpu_baseline(cfg, spec, args, xs_host):
    """The oracle as it is, on this host's cores, over a bounded sample of the
    same workload: consecutive steps on the first layer pool until the time
    budget is used."""
    import oracle
    import synth
    blocks = synth.expert_pool(cfg, 0)
    shared = synth.shared_block(cfg, 0)
    wr, b = synth.router(cfg, 0)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n_steps, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        x = xs_host[n_steps % len(xs_host)]
        oracle.layer_step(x, wr, b, cfg.k, blocks, shared, spec.d, spec.f, spec.wbits, spec.group)
        n_steps += 1
        tokens += x.shape[0]
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    el = time.perf_counter() - t0
    n_layers = len(cfg.layers) if len(set(cfg.layers)) > 1 else 1
    # a stack step runs every layer: scale the first layer's rate to the stack
    return {"value": tokens / el / n_layers, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} steps ({tokens} tokens) of the {cfg.name} layer step on the "
                      f"first layer pool, {el:.1f}s, float64 oracle with OpenMP"
                      + (f"; rate divided by the {n_layers} layers of a stack step"
                         if n_layers > 1 else "")}


if __name__ == "__main__":
    main()
