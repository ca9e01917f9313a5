#!/usr/bin/env python3
"""Throughput of the routed-expert layer step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens
already resident in HBM: per layer, route + top-k, union + permutation and hit
counters, then the expert math and the combine, all through the C ABI
(moe_layer_step) on one stream.

Default run (no --config): the headline is the largest single-GPU workload,
"stack8_draft": 8 GLM-5.2-shaped int4 MoE layers (d_model 6144, d_ff 2048,
256 routed + 1 shared expert, top-8, Zipf(1.1) router bias per layer) and an
int8 draft-head layer, 256 decode tokens per step, the layers chained through
a residual RMS norm; a step runs all 9 layers. Two sub-records follow it in
the same JSON line: "decode1" (one token, top-1: the single-token GEMV path,
8 layer pools rotated so the 256 MB Infinity Cache cannot serve a looped
working set) and "prefill4096" (4096 tokens, top-8, flat router bias: the
128-token matrix-core pass). --config NAME measures one workload alone.

Each workload is measured in three passes over the same steps:
  1. wall clock: W untimed warm-up steps, then exactly K steps between two
     torch.cuda.synchronize() calls, with no events or other instrumentation;
     `value` (tokens/s) and `ms_per_step` come from this pass only;
  2. per-step GPU time: the same steps again with one HIP event recorded on
     the stream between consecutive steps, for the p10 / p50 / p90 step times;
  3. per-kernel time: a sample of steps whose expert kernels take HIP events at
     their own start and end (hipExtLaunchKernelGGL on the library's stream),
     for the roofline of the dominant kernel: its algorithmic bytes (or flops)
     per launch over its mean duration. Event-taking launches cost the host
     microseconds each, which is why this pass is separate.
`roofline.measured_ceiling` is what the simplest kernel of the same kind
reaches on this GPU (a plain streaming read of the same bytes per launch, or
a loop of independent matrix-core products), beside the published peak.
`cpu_baseline` is the CPU oracle (float64, OpenMP) timed on this host on a
bounded sample of the headline workload.
"""
import argparse
import ctypes
import dataclasses
import glob
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s and expert-weight HBM GB/s (% of 8 TB/s peak) on 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense float16 matrix-core peak

# Arithmetic of each pass of the layer step
DTYPE_BY_PASS = {
    "router": "f32 (sums and sigmoid)",
    "gemv": "int4 codes x int16 activations as four base-16 digit planes (v_dot8c_i32_i4), "
            "int8 codes x two base-256 planes (v_dot4c_i32_i8): exact int32 per 32/16-column "
            "run, scaled in f32",
    "small": "f16 codes x f16 activations -> f32 accumulate (v_mfma_f32_16x16x32_f16), "
             "32-token items",
    "mfma": "f16 codes x f16 activations -> f32 accumulate (v_mfma_f32_16x16x32_f16), "
            "128-token items",
    "combine": "f32",
}
DTYPE = "int4/int8 weights; f16 MFMA and int16-digit dot products, f32 accumulate"

# Defaults of the sub-records of the headline run (independent of --steps,
# which applies to the headline)
SUB_RUNS = {"decode1": dict(steps=2000, warmup=400, layers=8, batches=16),
            "prefill4096": dict(steps=20, warmup=4, layers=2, batches=2)}
KERNEL_SAMPLES = 64   # layer steps whose kernels take events (pass 3), at least


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default=None,
                   help="measure this workload alone (tiny, decode1, decode64, prefill4096, "
                        "stack8_draft); default: stack8_draft with decode1 and prefill4096 "
                        "sub-records")
    p.add_argument("--tokens", type=int, default=None,
                   help="tokens per step instead of the workload's (e.g. a speculative "
                        "verify batch of 1 + drafts through the stack)")
    p.add_argument("--k", type=int, default=None, help="experts per token instead of the workload's")
    p.add_argument("--small-min", type=int, default=None,
                   help="experts with at least this many tokens take the 32-token matrix-core "
                        "pass (moe_forward_options.mfma_small_min_tokens; default: the library's)")
    p.add_argument("--group", type=int, default=None,
                   help="scale group of the int4 layers instead of the workload's (e.g. 64)")
    p.add_argument("--layers", type=int, default=8,
                   help="layer pools rotated over the steps (single-layer workloads)")
    p.add_argument("--batches", type=int, default=16, help="distinct token batches rotated")
    p.add_argument("--cpu-tokens", type=int, default=128,
                   help="tokens of the headline batch the CPU oracle runs through the stack")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="time budget of the CPU oracle on single-layer workloads")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-subrecords", action="store_true",
                   help="default run: the headline workload only")
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
    p.add_argument("--spec-drafts", default=None, metavar="D1,D2,..",
                   help="speculative decoding cycles on the stack workload: D draft steps "
                        "through the int8 draft layer, then a verify batch of 1 + D tokens "
                        "through the 8 int4 layers (moe_stack_forward), for each listed D")
    p.add_argument("--cache-slots", default=None,
                   help="comma-separated HBM slot counts: measure the Place stage (experts in "
                        "pinned host memory, an HBM cache of that many slots per layer) instead")
    return p.parse_args()


def say(msg):
    print(msg, file=sys.stderr, flush=True)


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
        vp = ctypes.c_void_p
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.L.hipEventDestroy.argtypes = [vp]
        self.L.hipEventRecord.argtypes = [vp, vp]
        self.L.hipMemcpyAsync.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]

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


# ---------------------------------------------------------------- environment

def _gpu_sysfs_dir(torch):
    """sysfs folder of cuda:0 (matched by PCI address), or None."""
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
    except Exception:
        return None
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            if os.path.basename(os.path.realpath(dev)).startswith(bdf):
                return dev
        except OSError:
            pass
    return None


def _current_mhz(path):
    """The active level of a pp_dpm_* file ("N: 2400Mhz *"), in MHz."""
    with open(path) as fh:
        for line in fh:
            if line.rstrip().endswith("*"):
                return int(line.split(":")[1].strip().lower().split("mhz")[0])
    return None


class ClockSampler:
    """Samples the GPU's current SCLK and MCLK (sysfs pp_dpm_sclk / pp_dpm_mclk)
    every few milliseconds on a side thread while a timed region runs."""

    def __init__(self, torch, period=0.005):
        self.dir = _gpu_sysfs_dir(torch)
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._t = None

    def __enter__(self):
        if self.dir:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append((_current_mhz(os.path.join(self.dir, "pp_dpm_sclk")),
                                     _current_mhz(os.path.join(self.dir, "pp_dpm_mclk"))))
            except (OSError, ValueError, IndexError):
                return
            time.sleep(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()

    def summary(self):
        s = [v for v in self.samples if v[0] is not None]
        if not s:
            return {"sclk_mhz": None, "mclk_mhz": None, "samples": 0,
                    "note": "GPU clock files not readable on this host"}
        sc = sorted(v[0] for v in s)
        mc = sorted(v[1] for v in s if v[1] is not None)
        return {"sclk_mhz": {"min": sc[0], "median": sc[len(sc) // 2], "max": sc[-1]},
                "mclk_mhz": ({"min": mc[0], "median": mc[len(mc) // 2], "max": mc[-1]}
                             if mc else None),
                "samples": len(s), "source": self.dir}


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cpu_model": model, "nproc": nproc, "cpu_count": os.cpu_count()}


def percentiles(v):
    import numpy as np
    v = np.asarray(v, np.float64)
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90)), "mean": float(v.mean()), "n": int(v.size)}


# ---------------------------------------------------------------- workloads

def build_workload(name, args, steps, warmup, layers, batches, dev, tokens=None, k=None,
                   group=None, small_min=None):
    """HBM-resident pools, routers and token batches of one workload, and the
    C-ABI calls of its steps with their arguments converted once."""
    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    base = synth.CONFIGS[name]
    if group is not None:
        base = dataclasses.replace(base, layers=tuple(
            dataclasses.replace(ls, group=group) if ls.wbits == 4 else ls for ls in base.layers))
    if tokens is not None:
        base = dataclasses.replace(base, n_tokens=tokens)
    if k is not None:
        base = dataclasses.replace(base, k=k)
    spec = base.layer
    stack = len(base.layers) > 1
    if stack:
        cfg, L_rot = base, len(base.layers)
    else:
        L_rot = layers
        cfg = dataclasses.replace(base, layers=(spec,) * L_rot)
    N, k, E, d, f = cfg.n_tokens, cfg.k, spec.n_experts, spec.d, spec.f
    nb = max(1, min(batches, steps + warmup))
    t0 = time.time()
    pools, routers = [], []
    for l in range(L_rot):
        ls = cfg.layers[l]
        blocks = synth.expert_pool(cfg, l)
        shared = synth.shared_block(cfg, l)
        pools.append(moe.DevicePool(d, f, E, ls.wbits, ls.group, blocks, shared, dev))
        del blocks
        wr, b = synth.router(cfg, l)
        routers.append((torch.from_numpy(wr).to(dev), torch.from_numpy(b).to(dev)))
        say(f"[bench] {name}: layer pool {l + 1}/{L_rot} resident")
    tok_cfg = dataclasses.replace(cfg, n_tokens=N * nb)
    xs_host = synth.tokens(tok_cfg).reshape(nb, N, d)
    xs = torch.from_numpy(xs_host).to(dev)
    w = dict(
        ids=torch.empty((N, k), dtype=torch.int32, device=dev),
        w=torch.empty((N, k), dtype=torch.float32, device=dev),
        union_ids=torch.empty(E, dtype=torch.int32, device=dev),
        n_union=torch.empty(1, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(N * k, dtype=torch.int32, device=dev),
        counters=torch.zeros((L_rot, E), dtype=torch.int64, device=dev),
        y=torch.empty((N, d), dtype=torch.float32, device=dev),
        hbuf=torch.empty((N, d), dtype=torch.float32, device=dev),   # residual stream
        abuf=torch.empty((N, d), dtype=torch.float32, device=dev),   # normalised layer input
    )
    ws_bytes = max(moe.layer_step_workspace_size(p.desc, N, k) for p in pools)
    w["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return dict(name=name, cfg=cfg, base=base, spec=spec, stack=stack, L_rot=L_rot, N=N, k=k, E=E,
                d=d, f=f, nb=nb, pools=pools, routers=routers, xs=xs, xs_host=xs_host,
                bufs=w, ws_bytes=ws_bytes, small_min=small_min, setup_s=time.time() - t0)


class Runner:
    """Launches the steps of a workload through the C ABI: moe_layer_step for
    a single layer; for a stack, moe_stack_forward (or, when events or
    per-layer callbacks are asked for, moe_residual_rmsnorm and
    moe_layer_step per layer)."""

    def __init__(self, wl, hip, torch):
        import int4_routed_expert_gemv_amd as moe
        self.wl, self.hip = wl, hip
        self.moe = moe
        self.L = moe.lib()
        vp = ctypes.c_void_p
        self.vp = vp
        self.stream = vp(torch.cuda.current_stream().cuda_stream)
        b = wl["bufs"]
        self.base_opts = None
        if wl["small_min"] is not None:
            self.base_opts = moe.ForwardOptions()
            self.base_opts.mfma_small_min_tokens = wl["small_min"]
        N, d, k = wl["N"], wl["d"], wl["k"]

        def args(l, x):
            wr, bias = wl["routers"][l]
            return (ctypes.byref(wl["pools"][l].desc), vp(x.data_ptr()), N, d, vp(wr.data_ptr()),
                    vp(bias.data_ptr()), k, vp(b["ids"].data_ptr()), vp(b["w"].data_ptr()),
                    vp(b["union_ids"].data_ptr()), vp(b["n_union"].data_ptr()),
                    vp(b["offsets"].data_ptr()), vp(b["perm"].data_ptr()),
                    vp(b["counters"][l].data_ptr()), vp(b["y"].data_ptr()),
                    vp(b["ws"].data_ptr()), wl["ws_bytes"], self.stream)

        if wl["stack"]:
            self.layer_args = [args(l, b["abuf"]) for l in range(wl["L_rot"])]
            # the timed steps run the whole stack in one moe_stack_forward call;
            # calibration and the per-kernel event pass take its layers one
            # moe_layer_step at a time (the same kernels and outputs, bit for
            # bit, except that the stack call joins each combine with the next
            # residual norm)
            self.stack_layers = moe.layer_descs(
                [(wl["pools"][l].desc, wl["routers"][l][0], wl["routers"][l][1],
                  b["counters"][l]) for l in range(wl["L_rot"])])
            nbytes = moe.stack_workspace_size(self.stack_layers, N, k)
            if nbytes <= 0:
                raise RuntimeError("moe_stack_workspace_size rejected the stack")
            self.stack_ws = torch.empty(nbytes, dtype=torch.uint8, device=b["y"].device)
        else:
            # one plan per (layer pool, batch) pair: step s takes plan s % n_plan
            self.plans = [args(p % wl["L_rot"], wl["xs"][p % wl["nb"]])
                          for p in range(wl["L_rot"] * wl["nb"])]

    def layer(self, a, opt):
        o = opt if opt is not None else self.base_opts
        rc = self.L.moe_layer_step(*a, None if o is None else ctypes.byref(o))
        if rc:
            raise RuntimeError(f"moe_layer_step failed with status {rc}")

    def step(self, s, evs=None, sync_layers=None):
        """Step s; evs: per layer, a ForwardOptions with events (or None);
        sync_layers(l): called after each layer (calibration only)."""
        wl = self.wl
        if not wl["stack"]:
            self.layer(self.plans[s % len(self.plans)], evs[0] if evs else None)
            if sync_layers:
                sync_layers(s % len(self.plans))
            return
        b, vp = wl["bufs"], self.vp
        x = wl["xs"][s % wl["nb"]]
        rc = self.hip.L.hipMemcpyAsync(vp(b["hbuf"].data_ptr()), vp(x.data_ptr()),
                                       x.numel() * 4, 3, self.stream)
        if evs is None and sync_layers is None:
            rc |= self.L.moe_stack_forward(self.stack_layers, wl["L_rot"], wl["N"], wl["k"],
                                           ctypes.c_float(1e-6), vp(b["hbuf"].data_ptr()), None,
                                           vp(self.stack_ws.data_ptr()), self.stack_ws.numel(),
                                           self.stream)
            if rc:
                raise RuntimeError(f"stack step failed with status {rc}")
            return
        for l in range(wl["L_rot"]):
            rc |= self.L.moe_residual_rmsnorm(vp(b["hbuf"].data_ptr()),
                                              vp(b["y"].data_ptr()) if l else None,
                                              vp(b["abuf"].data_ptr()), wl["N"], wl["d"],
                                              ctypes.c_float(1e-6), self.stream)
            if rc:
                raise RuntimeError(f"stack step failed with status {rc}")
            self.layer(self.layer_args[l], evs[l] if evs else None)
            if sync_layers:
                sync_layers((s % wl["nb"], l))


def calibrate(wl, runner, torch, small_min):
    """Which experts each (layer, batch) step streams and on which pass (the
    library's default thresholds): experts with at least 32 tokens go to the
    128-token matrix-core pass, those with at least small_min (default 1) to
    the 32-token pass, the rest (and every expert of a batch of at most 2
    tokens) to the GEMV; fewer than 32 items of 128 tokens, or fewer than
    32 * 128 assignments in the batch, join the 32-token pass; a
    128-token group's remainder of at most 32 tokens past a full item goes to
    the 32-token pass. The shared expert counts as an expert of N tokens."""
    import numpy as np
    MFMA_MIN, MIN_BIG_ITEMS, GEMV_BATCH = 32, 32, 2
    SMALL_MIN = small_min if small_min is not None else 1
    N, d, f = wl["N"], wl["d"], wl["f"]
    b = wl["bufs"]
    calib = {}

    def pass_of(T, mfma_ok):
        T = np.asarray(T)
        big = (T >= MFMA_MIN) & mfma_ok
        small = ~big & (T >= SMALL_MIN) & mfma_ok & (N > GEMV_BATCH or small_min is not None)
        if big.any() and (np.sum((T[big] + 127) // 128) < MIN_BIG_ITEMS or
                          N * wl["k"] < MIN_BIG_ITEMS * 128):
            small, big = small | big, np.zeros_like(big)
        return np.where(big, 1, np.where(small, 2, 0))

    def record(key):
        torch.cuda.synchronize()
        l = key[1] if wl["stack"] else key % wl["L_rot"]
        ls = wl["cfg"].layers[l]
        # the matrix-core passes take int4 and int8 layers alike (every
        # supported shape has whole 128- or 64-column units)
        mfma_ok = True
        nu = int(b["n_union"].item())
        uid = b["union_ids"][:nu].cpu().numpy()
        off = b["offsets"].cpu().numpy()
        T = np.concatenate([off[uid + 1] - off[uid], [N]])  # routed, then shared
        ps = pass_of(T, mfma_ok)
        c = dict(union=nu, wbits=ls.wbits, group=ls.group, layer=l)
        for name, code in (("gemv", 0), ("mfma", 1), ("small", 2)):
            c[name + "_experts"] = int((ps == code).sum())
            c[name + "_tokens"] = int(T[ps == code].sum())
        if mfma_ok and (N > GEMV_BATCH or small_min is not None) and SMALL_MIN > 0:
            r = T % 128
            rem = (ps == 1) & (T > 128) & (r > 0) & (r <= 32)
            c["mfma_tokens"] -= int(r[rem].sum())
            c["small_tokens"] += int(r[rem].sum())
            c["small_experts"] += int(rem.sum())
        calib[key] = c

    n = wl["nb"] if wl["stack"] else len(runner.plans)
    for s in range(n):
        runner.step(s, sync_layers=record)
    torch.cuda.synchronize()
    return calib


def layer_sizes(moe, d, f, c):
    """(whole block bytes, gate + up bytes) of one expert of layer record c."""
    bb = moe.block_bytes(d, f, c["wbits"], c["group"])
    q_gu = f * d * c["wbits"] // 8
    s_gu = f * (d // c["group"] if c["group"] else 1) * 4
    return bb, 2 * (q_gu + s_gu)


KERNEL_LABELS = {
    "gemv": ("gemv_kernel<gate/up> (expert gate and up projections, SiLU product)",
             "moe::gemv_kernel<true, {wb}, 1"),
    "small": ("mfma_kernel<gate/up, 32 tokens> (small-group gate and up on the matrix cores)",
              "moe::mfma_kernel<true, {wb}, 2"),
    "mfma": ("mfma_kernel<gate/up, 128 tokens> (grouped GEMM of gate and up, SiLU product)",
             "moe::mfma_kernel<true, {wb}, 8"),
}


def measure(wl, args, steps, warmup, hip, torch, traffic_key):
    """The three passes (wall clock, per-step events, per-kernel events) over
    one workload; returns its record (no cpu_baseline)."""
    import numpy as np

    import int4_routed_expert_gemv_amd as moe
    name, N, k, d, f, E = wl["name"], wl["N"], wl["k"], wl["d"], wl["f"], wl["E"]
    stack = wl["stack"]
    runner = Runner(wl, hip, torch)
    calib = calibrate(wl, runner, torch, wl["small_min"])
    mean_union = float(np.mean([c["union"] for c in calib.values()]))
    n_plan = wl["nb"] if stack else len(runner.plans)

    def keys_of(s):
        """calibration keys of the layers step s runs"""
        if stack:
            return [(s % wl["nb"], l) for l in range(wl["L_rot"])]
        return [s % n_plan]

    # ---- pass 1: wall clock, nothing but the steps ----------------------------
    for s in range(warmup):
        runner.step(s)
    torch.cuda.synchronize()
    say(f"[bench] {name}: setup {wl['setup_s']:.1f}s, mean union {mean_union:.1f}; "
        f"timing {steps} steps")
    K = steps
    with ClockSampler(torch) as clocks:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            runner.step(warmup + s)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / K * 1e3

    # ---- pass 2: per-step GPU time --------------------------------------------
    evs = [hip.event() for _ in range(K + 1)]
    torch.cuda.synchronize()
    for s in range(K):
        hip.L.hipEventRecord(evs[s], runner.stream)
        runner.step(warmup + s)
    hip.L.hipEventRecord(evs[K], runner.stream)
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(evs[s], evs[s + 1]) for s in range(K)]
    for e in evs:
        hip.L.hipEventDestroy(e)

    # ---- pass 3: per-kernel events on a sample of steps ------------------------
    # the same K steps once more, every `every`-th one with events on its
    # expert kernels and the others plain, so that the GPU stays as busy as
    # in pass 1 (back-to-back instrumented steps would leave it idle between
    # the short decode steps, and kernels started from idle run longer)
    per_step_layers = wl["L_rot"] if stack else 1
    n_samp = max(1, min(K, -(-KERNEL_SAMPLES // per_step_layers)))
    every = max(1, K // n_samp)
    samp_steps = [warmup + s for s in range(0, every * n_samp, every)]
    fo = {}
    for s in samp_steps:
        fo[s] = [moe.ForwardOptions(*[hip.event() for _ in range(12)], 0,
                                    wl["small_min"] if wl["small_min"] is not None else 0)
                 for _ in range(per_step_layers)]
    ev_fields = [n for n, t in moe.ForwardOptions._fields_ if t is ctypes.c_void_p]
    torch.cuda.synchronize()
    for s in range(warmup, warmup + max(K, every * n_samp)):
        runner.step(s, evs=fo.get(s))
    torch.cuda.synchronize()
    fo = [fo[s] for s in samp_steps]

    def ms(e, a, b):
        try:
            return hip.elapsed_ms(getattr(e, a), getattr(e, b))
        except AssertionError:  # the kernel was not launched in that step
            return None

    # per pass and weight width: (algorithmic gate/up bytes, flops, gate/up
    # time, down bytes, down time) of every sampled launch
    launches = {}
    for s, opts in zip(samp_steps, fo):
        for key, o in zip(keys_of(s), opts):
            c = calib[key]
            bb, gub = layer_sizes(moe, d, f, c)
            for pname, pre in (("gemv", ""), ("mfma", "mfma_"), ("small", "small_")):
                t_gu = ms(o, pre + "gateup_start", pre + "gateup_end")
                t_dn = ms(o, pre + "down_start", pre + "down_end")
                if t_gu is None or c[pname + "_experts"] == 0:
                    continue
                launches.setdefault((pname, c["wbits"]), []).append(
                    (c[pname + "_experts"] * gub, 4.0 * d * f * c[pname + "_tokens"], t_gu,
                     c[pname + "_experts"] * (bb - gub), t_dn))
    for opts in fo:
        for o in opts:
            for fld in ev_fields:
                hip.L.hipEventDestroy(getattr(o, fld))

    passes = {}
    for (pname, wb), v in launches.items():
        v = np.asarray([(a, b_, c_, d_, e_ if e_ is not None else np.nan) for a, b_, c_, d_, e_ in v])
        t_gu = v[:, 2].mean() / 1e3
        t_dn = np.nanmean(v[:, 4]) / 1e3 if np.isfinite(v[:, 4]).any() else None
        gu_b, fl, dn_b = v[:, 0].mean(), v[:, 1].mean(), v[:, 3].mean()
        passes[f"{pname}_int{wb}"] = {
            "kernel": KERNEL_LABELS[pname][1].format(wb=wb), "launches": int(len(v)),
            "avg_launch_us": t_gu * 1e6, "bytes_per_launch": gu_b, "achieved_GBps": gu_b / 1e9 / t_gu,
            "flops_per_launch": fl, "achieved_TFLOPs": fl / 1e12 / t_gu,
            "total_ms_in_sample": float(v[:, 2].sum()),
            "down_avg_launch_us": t_dn * 1e6 if t_dn else None,
            "down_GBps": dn_b / 1e9 / t_dn if t_dn else None,
            "dtype": DTYPE_BY_PASS[pname]}

    # algorithmic bytes of the timed steps (pass 1)
    expert_bytes = router_bytes = 0
    for s in range(K):
        for key in keys_of(warmup + s):
            c = calib[key]
            bb, _ = layer_sizes(moe, d, f, c)
            expert_bytes += (c["union"] + 1) * bb
            router_bytes += E * d * 4 + E * 4

    roof = None
    if passes:
        # the dominant kernel: the gate/up kernel with the most time in the sample
        top = max(passes, key=lambda n: passes[n]["total_ms_in_sample"])
        pz = passes[top]
        pname = top.rsplit("_int", 1)[0]
        if pname == "mfma":
            roof = {"bound": "mfma", "achieved": pz["achieved_TFLOPs"],
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": pz["achieved_TFLOPs"] / MFMA_F16_PEAK_TFLOPS}
        else:
            roof = {"bound": "hbm", "achieved": pz["achieved_GBps"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": pz["achieved_GBps"] / HBM_PEAK_GBS}
        roof["traffic"] = measured_traffic(traffic_key, pz["kernel"]) if traffic_key else None
        roof["kernel"] = KERNEL_LABELS[pname][0] + f", int{top.split('int')[1]} weights"
        roof["kernel_symbol"] = pz["kernel"]
        roof["avg_launch_us"] = pz["avg_launch_us"]
        roof["algorithmic_per_launch"] = (pz["flops_per_launch"] if pname == "mfma"
                                          else pz["bytes_per_launch"])
        roof["timing"] = (f"HIP events taken by the kernel's own dispatches on the library's "
                          f"stream, {pz['launches']} launches: every {every}th of the timed "
                          f"steps, run again after the timed region")
        roof["passes"] = passes
        roof["measured_ceiling"] = measured_ceiling(moe, hip, torch, roof["bound"],
                                                    pz["bytes_per_launch"], roof["achieved"])
    steps_pct = percentiles(step_ms)
    rec = {
        "metric": METRIC,
        "value": N * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "step_ms_events": steps_pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "dtype_by_pass": DTYPE_BY_PASS,
        "data": "synthetic",
        "config": {
            "workload": wl["workload"],
            "n_tokens": N, "k": k, "d_model": d, "d_ff": f, "n_experts": E,
            "wbits": [ls.wbits for ls in wl["cfg"].layers] if stack else wl["spec"].wbits,
            "group": wl["spec"].group, "layers_per_step": wl["L_rot"] if stack else 1,
            "layer_pools": wl["L_rot"], "token_batches": wl["nb"], "mean_union": mean_union,
        },
        "expert_GBps": expert_bytes / 1e9 / elapsed,
        "expert_frac_of_peak": expert_bytes / 1e9 / elapsed / HBM_PEAK_GBS,
        "step_GBps": (expert_bytes + router_bytes) / 1e9 / elapsed,
        "algorithmic_bytes_per_step": (expert_bytes + router_bytes) / K,
        "clocks": clocks.summary(),
        "roofline": roof,
    }
    if stack:
        rec["layer_tokens_per_s"] = N * wl["L_rot"] * K / elapsed
    say(f"[bench] {name}: {rec['value']:.1f} tokens/s, {ms_per_step * 1e3:.1f} us/step "
        f"(events p50 {steps_pct['p50'] * 1e3:.1f} us)"
        + (f"; {roof['kernel_symbol']} {roof['avg_launch_us']:.1f} us, frac {roof['frac']:.3f}"
           if roof else ""))
    return rec


def workload_label(wl, args_like):
    cfg, base = wl["cfg"], wl["base"]
    return (f"{cfg.name}: {base.description}" +
            ("" if wl["stack"] else f"; {wl['L_rot']} layer pools rotated") +
            (f"; int4 scale groups of {args_like.get('group')}" if args_like.get("group") else "") +
            (f"; {wl['N']} tokens per step" if args_like.get("tokens") is not None else "") +
            (f"; top-{wl['k']}" if args_like.get("k") is not None else ""))


def run_workload(name, args, steps, warmup, layers, batches, hip, torch, dev, tokens=None, k=None,
                 group=None, small_min=None, keep=False):
    wl = build_workload(name, args, steps, warmup, layers, batches, dev, tokens=tokens, k=k,
                        group=group, small_min=small_min)
    wl["workload"] = workload_label(wl, dict(group=group, tokens=tokens, k=k))
    plain = tokens is None and k is None
    traffic_key = (name if group is None else f"{name}_g{group}") if plain else None
    rec = measure(wl, args, steps, warmup, hip, torch, traffic_key)
    if keep:
        return rec, wl
    del wl
    torch.cuda.empty_cache()
    return rec, None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.cache_slots:
        cache_bench(args)
        return
    if args.cache_stack:
        cache_stack_bench(args)
        return
    if args.spec_drafts:
        spec_bench(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    name = args.config or "stack8_draft"
    rec, wl = run_workload(name, args, args.steps, args.warmup, args.layers, args.batches, hip,
                           torch, dev, tokens=args.tokens, k=args.k, group=args.group,
                           small_min=args.small_min, keep=not args.no_cpu_baseline)
    cpu_inputs = None
    if wl is not None:
        cpu_inputs = (wl["cfg"], wl["stack"], wl["xs_host"])
        del wl
        torch.cuda.empty_cache()
    if args.config is None and not args.no_subrecords:
        subs = {}
        for sub, kw in SUB_RUNS.items():
            r, _ = run_workload(sub, args, kw["steps"], kw["warmup"], kw["layers"], kw["batches"],
                                hip, torch, dev)
            for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline",
                        "dtype_by_pass", "data", "unit"):
                r.pop(key, None)
            subs[sub] = r
        rec["sub_records"] = subs
    rec["host"] = host_info()
    rec["cpu_baseline"] = None
    if cpu_inputs is not None:
        rec["cpu_baseline"] = cpu_baseline(*cpu_inputs, args)
    print(json.dumps(rec), flush=True)


def cache_bench(args):
    """Place and Overlap stages: each layer's routed experts in pinned host
    memory, an HBM cache of C slots per layer (moe_cache_*, least recently
    used replacement). A step routes the batch (moe_route_union) and copies
    the union to the host; then either ("place") places it, the missing
    blocks copied on a second stream, and runs the expert math through the
    slot table, or ("overlap", moe_cache_forward) runs the resident experts'
    math while the missing blocks are copied, then the rest. Reported per
    slot count and mode: tokens/s, the hit rate over the timed steps and the
    bytes copied per token next to the L*k*S*(1-h) estimate (here L = 1
    layer per step); and the step time with every expert resident."""
    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    dev = torch.device("cuda:0")
    base = synth.CONFIGS[args.config or "decode1"]
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

    def resident_step_ms():
        """the same steps with every expert resident (the compute alone)"""
        pools = [moe.DevicePool(d, f, E, spec.wbits, spec.group, synth.expert_pool(cfg, l),
                                synth.shared_block(cfg, l), dev) for l in range(L_rot)]

        def run(s_):
            ly, pl = layers[s_ % L_rot], pools[s_ % L_rot]
            x = xs[s_ % nb]
            moe.route_union(x, ly["wr"], ly["b"], k, ids, w, uid, nu, off, perm, cnt, ws)
            moe.expert_forward(pl.desc, x, k, w, uid, nu, off, perm, y, ws)

        for s_ in range(min(args.warmup, 50)):
            run(s_)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            run(s_)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps * 1e3
        del pools
        torch.cuda.empty_cache()
        return el

    t_res = resident_step_ms()
    points = []
    for C in [int(c) for c in args.cache_slots.split(",")]:
        for mode in ("place", "overlap"):
            caches = [moe.ExpertCache(ly["desc"], C, ly["host"], dev) for ly in layers]

            def run(s_):
                ly, cache = layers[s_ % L_rot], caches[s_ % L_rot]
                x = xs[s_ % nb]
                moe.route_union(x, ly["wr"], ly["b"], k, ids, w, uid, nu, off, perm, cnt, ws)
                n = int(nu.item())
                union = uid[:n].cpu().numpy()
                if mode == "overlap":
                    # Place + Overlap: resident experts compute while the
                    # missing ones are copied in
                    cache.forward(x, k, w, uid, nu, off, perm, union, y, ws,
                                  copy_stream=copy_stream)
                else:
                    cache.place(union, copy_stream=copy_stream)
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
            points.append({"slots": C, "mode": mode, "tokens_per_s": tok / el,
                           "ms_per_step": el / args.steps * 1e3,
                           "hit_rate": hr, "misses_per_step": misses / args.steps,
                           "copied_bytes_per_token": misses * block / tok,
                           "estimate_bytes_per_token": k * block * (1 - hr),
                           "copied_GBps": misses * block / el / 1e9})
            print(f"[cache bench] {C} slots, {mode}: {points[-1]}", file=sys.stderr, flush=True)
            for c in caches:
                c.close()
            del caches
    print(json.dumps({"metric": "layer-step tokens/s with experts placed from pinned host memory "
                                "into an HBM cache (Place stage, without and with Overlap)",
                      "resident_ms_per_step": t_res,
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


def spec_bench(args):
    """Speculative decoding through the same kernels (Colibri README,
    "Speculative decoding, honestly"): per cycle, D draft steps of one token
    each through the int8 draft-head layer (g_i = g_(i-1) + draft(rms(g_(i-1)))),
    then the verify batch [g_0 .. g_D] through the 8 int4 layers, all with
    moe_stack_forward. Reported per D: the cycle time, its draft and verify
    parts, and the tokens per second if every draft were accepted, next to
    plain one-token decode through the 8 int4 layers (D = 0). Acceptance
    itself needs a trained model and is not measured."""
    import numpy as np
    import torch

    import int4_routed_expert_gemv_amd as moe
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Ds = sorted({int(v) for v in args.spec_drafts.split(",")} | {0})
    wl = build_workload("stack8_draft", args, 1, 0, 1, 1, dev)
    k, d, L = wl["k"], wl["d"], wl["L_rot"]
    descs = [(wl["pools"][l].desc, wl["routers"][l][0], wl["routers"][l][1], None)
             for l in range(L)]
    draft = moe.layer_descs(descs[L - 1:])
    main = moe.layer_descs(descs[:L - 1])
    maxD = max(Ds)
    ws = torch.empty(max(moe.stack_workspace_size(draft, 1, k),
                         moe.stack_workspace_size(main, 1 + maxD, k)), dtype=torch.uint8,
                     device=dev)
    x0 = torch.from_numpy(synth.tokens(dataclasses.replace(wl["cfg"], n_tokens=1))).to(dev)
    g = torch.empty((1 + maxD, d), dtype=torch.float32, device=dev)
    hip = Hip()
    evs = [hip.event() for _ in range(3)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def cycle(D, ev=False):
        g[0].copy_(x0[0])
        if ev:
            hip.L.hipEventRecord(evs[0], stream)
        for i in range(1, D + 1):
            g[i].copy_(g[i - 1])
            moe.stack_forward(draft, g[i:i + 1], k, ws)
        if ev:
            hip.L.hipEventRecord(evs[1], stream)
        moe.stack_forward(main, g[:D + 1], k, ws)
        if ev:
            hip.L.hipEventRecord(evs[2], stream)

    points = []
    for D in Ds:
        for _ in range(max(2, args.warmup)):
            cycle(D)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            cycle(D)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        dr, vf = [], []
        for _ in range(min(args.steps, 20)):
            cycle(D, ev=True)
            torch.cuda.synchronize()
            dr.append(hip.elapsed_ms(evs[0], evs[1]) if D else 0.0)
            vf.append(hip.elapsed_ms(evs[1], evs[2]))
        pt = {"drafts": D, "verify_tokens": D + 1, "ms_per_cycle": ms,
              "draft_ms": float(np.median(dr)), "verify_ms": float(np.median(vf)),
              "tokens_per_s_all_accepted": (D + 1) / ms * 1e3}
        points.append(pt)
        say(f"[spec] {pt}")
    base = points[0]["ms_per_cycle"]
    for pt in points:
        pt["speedup_all_accepted"] = pt["tokens_per_s_all_accepted"] / (1e3 / base)
    print(json.dumps({"metric": "speculative decoding cycles through the layer stack: D draft "
                                "steps on the int8 draft layer + a verify batch of 1 + D tokens "
                                "on the 8 int4 layers",
                      "unit": "ms per cycle", "n_gpus": 1, "steps": args.steps,
                      "data": "synthetic",
                      "config": {"workload": "stack8_draft layers: 8 int4 GLM-5.2-shaped layers "
                                             "(top-8, Zipf(1.1) bias) + the int8 draft layer",
                                 "k": k, "d_model": d},
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


def cpu_baseline(cfg, stack, xs_host, args):
    """The oracle as it stands (plain C, float64 arithmetic, OpenMP over
    independent rows), timed on this host's cores over a bounded sample of
    the same workload. A stack: the first --cpu-tokens tokens of the first
    batch through every layer (RMS norm, route, top-k, union, counters,
    experts, combine per layer); each layer's inputs are drawn from the seed
    before its timed part. A single layer: consecutive steps on the first
    layer pool for --cpu-seconds."""
    import numpy as np

    import oracle
    import synth
    threads = oracle.threads()
    if stack:
        T = max(1, min(args.cpu_tokens, cfg.n_tokens))
        h = xs_host[0][:T].astype(np.float64)
        busy = 0.0
        for l, ls in enumerate(cfg.layers):
            blocks = synth.expert_pool(cfg, l)
            shared = synth.shared_block(cfg, l)
            wr, b = synth.router(cfg, l)
            t0 = time.perf_counter()
            a = oracle.rms_normalize(h, 1e-6)
            ref = oracle.layer_step(a, wr, b, cfg.k, blocks, shared, ls.d, ls.f, ls.wbits,
                                    ls.group)
            h = h + ref["y"]
            busy += time.perf_counter() - t0
            del blocks
            say(f"[bench] cpu oracle: layer {l + 1}/{len(cfg.layers)}, {busy:.1f}s so far")
        return {"value": T / busy, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "arith": "float64",
                "sample": f"{T} of the {cfg.n_tokens} tokens of one {cfg.name} batch through all "
                          f"{len(cfg.layers)} layers (oracle: RMS norm, router, top-k, union, "
                          f"counters, experts, combine per layer), {busy:.1f}s of oracle time; "
                          f"float64 oracle with OpenMP"}
    spec = cfg.layers[0]
    blocks = synth.expert_pool(cfg, 0)
    shared = synth.shared_block(cfg, 0)
    wr, b = synth.router(cfg, 0)
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
            "arith": "float64",
            "sample": f"{n_steps} steps ({tokens} tokens) of the {cfg.name} layer step on the "
                      f"first layer pool, {el:.1f}s, float64 oracle with OpenMP"}


if __name__ == "__main__":
    main()
