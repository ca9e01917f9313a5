#!/usr/bin/env python3
"""Throughput of the routed-expert layer step on one MI355X.

A step is one pass of the whole layer step over one batch: route + top-k,
union + permutation, hit counters, expert math + combine (four C-ABI calls,
all on one stream). Inputs are synthetic and already resident in HBM.

Default workload ("decode1"): one GLM-5.2-shaped decode layer (d_model 6144,
d_ff 2048, 256 routed + 1 shared int4 experts with float32 scales per 128,
top-1, 1 token per step). Successive steps walk through --layers independently
drawn layer pools (each its own router and experts), as a decode pass walks
through a model's layers, so the 256 MB Infinity Cache cannot serve a
repeated working set.

Prints one JSON line. `roofline` is for the gate/up GEMV kernel (the largest
kernel of a decode step), timed with HIP events recorded on the library's
stream around that kernel in every timed step. `cpu_baseline` is the CPU
oracle timed on this host on a bounded sample of the same workload.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--config", default="decode1")
    p.add_argument("--layers", type=int, default=8, help="layer pools rotated over the steps")
    p.add_argument("--batches", type=int, default=16, help="distinct token batches rotated")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


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
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.CONFIGS[args.config]
    spec = base.layer
    L_rot = args.layers
    cfg = dataclasses.replace(base, layers=(spec,) * L_rot)
    N, k, E, d, f = cfg.n_tokens, cfg.k, spec.n_experts, spec.d, spec.f
    A = N * k
    nb = max(1, min(args.batches, args.steps + args.warmup))
    t_setup = time.time()

    # --- inputs resident in HBM -------------------------------------------
    pools, routers = [], []
    for l in range(L_rot):
        blocks = synth.expert_pool(cfg, l)
        shared = synth.shared_block(cfg, l)
        pools.append(moe.DevicePool(d, f, E, spec.wbits, spec.group, blocks, shared, dev))
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
    ws_bytes = moe.workspace_size(pools[0].desc, N, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # --- raw C-ABI calls with their arguments converted once ---------------
    Lb = moe.lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    hip = Hip()

    def step_args(s):
        l, bi = s % L_rot, s % nb
        x = xs[bi]
        wr, b = routers[l]
        route = (vp(x.data_ptr()), N, d, vp(wr.data_ptr()), vp(b.data_ptr()), E, k,
                 vp(ids.data_ptr()), vp(w.data_ptr()), vp(ws.data_ptr()), ws_bytes, stream)
        uni = (vp(ids.data_ptr()), N, k, E, vp(union_ids.data_ptr()), vp(n_union.data_ptr()),
               vp(offsets.data_ptr()), vp(perm.data_ptr()), stream)
        hit = (vp(ids.data_ptr()), N, k, E, vp(counters[l].data_ptr()), stream)
        fwd = (ctypes.byref(pools[l].desc), vp(x.data_ptr()), N, k, vp(w.data_ptr()),
               vp(union_ids.data_ptr()), vp(n_union.data_ptr()), vp(offsets.data_ptr()),
               vp(perm.data_ptr()), vp(y.data_ptr()), vp(ws.data_ptr()), ws_bytes, stream)
        return route, uni, hit, fwd

    plans = [step_args(s) for s in range(L_rot * nb)]
    n_plan = len(plans)

    def run(s, ev=None):
        route, uni, hit, fwd = plans[s % n_plan]
        rc = Lb.moe_route_topk(*route)
        rc |= Lb.moe_union(*uni)
        rc |= Lb.moe_hit_count(*hit)
        if ev is None:
            rc |= Lb.moe_expert_forward(*fwd)
        else:
            rc |= Lb.moe_expert_forward_ex(*fwd, ctypes.byref(ev))
        if rc:
            raise RuntimeError(f"layer step failed with status {rc}")

    # union size of every (layer, batch) step: the experts a step streams
    u_of = []
    for s in range(n_plan):
        run(s)
        torch.cuda.synchronize()
        u_of.append(int(n_union.item()))
    for _ in range(args.warmup):
        run(_)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.time() - t_setup:.1f}s; mean union {np.mean(u_of):.1f}",
          file=sys.stderr, flush=True)

    # --- timed region -------------------------------------------------------
    K = args.steps
    evs = [moe.ForwardOptions(*[hip.event() for _ in range(8)], 0) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        run(args.warmup + s, evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    gu_ms = [hip.elapsed_ms(e.gateup_start, e.gateup_end) for e in evs]
    dn_ms = [hip.elapsed_ms(e.down_start, e.down_end) for e in evs]
    for e in evs:
        for h in (e.gateup_start, e.gateup_end, e.down_start, e.down_end, e.mfma_gateup_start,
                  e.mfma_gateup_end, e.mfma_down_start, e.mfma_down_end):
            hip.L.hipEventDestroy(h)

    # --- algorithmic bytes ---------------------------------------------------
    bb = moe.block_bytes(d, f, spec.wbits, spec.group)
    q_gu = f * d * spec.wbits // 8
    s_gu = f * (d // spec.group if spec.group else 1) * 4
    gu_bytes_per_expert = 2 * (q_gu + s_gu)          # gate + up codes and scales
    dn_bytes_per_expert = bb - gu_bytes_per_expert
    steps_u = [u_of[(args.warmup + s) % n_plan] for s in range(K)]
    n_exp = [u + 1 for u in steps_u]                 # union + shared expert
    gu_bytes = [n * gu_bytes_per_expert for n in n_exp]
    expert_bytes = sum(n * bb for n in n_exp)
    router_bytes = E * d * 4 + E * 4
    gu_avg_ms = float(np.mean(gu_ms))
    gu_achieved = (float(np.mean(gu_bytes)) / 1e9) / (gu_avg_ms / 1e3)
    dn_avg_ms = float(np.mean(dn_ms))
    dn_achieved = (float(np.mean([n * dn_bytes_per_expert for n in n_exp])) / 1e9) / (dn_avg_ms / 1e3)
    ms_per_step = elapsed / K * 1e3
    tokens_per_s = N * K / elapsed
    expert_gbs = expert_bytes / 1e9 / elapsed

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
        "dtype": "int4xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {base.description}; {L_rot} layer pools rotated",
            "n_tokens": N, "k": k, "d_model": d, "d_ff": f, "n_experts": E,
            "wbits": spec.wbits, "group": spec.group, "layer_pools": L_rot,
            "mean_union": float(np.mean(steps_u)),
        },
        "expert_GBps": expert_gbs,
        "expert_frac_of_peak": expert_gbs / HBM_PEAK_GBS,
        "step_GBps": (expert_bytes + K * router_bytes) / 1e9 / elapsed,
        "roofline": {
            "kernel": "gemv_kernel<gate/up> (expert gate and up projections, SiLU product)",
            "bound": "hbm",
            "achieved": gu_achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_achieved / HBM_PEAK_GBS,
            "traffic": None,
            "avg_launch_us": gu_avg_ms * 1e3,
            "bytes_per_launch": float(np.mean(gu_bytes)),
            "down_kernel_GBps": dn_achieved,
            "down_avg_launch_us": dn_avg_ms * 1e3,
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, spec, args, xs.cpu().numpy())
    print(json.dumps(result), flush=True)


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
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} steps ({tokens} tokens) of the {cfg.name} layer step on the "
                      f"first layer pool, {el:.1f}s, float64 oracle with OpenMP"}


if __name__ == "__main__":
    main()
