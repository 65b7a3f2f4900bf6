"""Benchmark of the fused MXFP4 GEMM + epilogue hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic DiT inputs:
online MXFP4 quantisation of each layer's activations, then the fused FP4
GEMM with its epilogue, for every linear of the workload.  Inputs are
resident in HBM before the timed region; activation buffers rotate over
several copies (more than the 256 MB last-level cache) so the quantiser reads
HBM, while the packed weights stay cache-warm as they would in serving.

Workloads (seeded synthetic tensors, random-init weights):
  dit_1k_linears (default)  one 1K image (4096 tokens): QKV 3072->9216 with
                            per-head RMSNorm hd 128 on Q,K; QKV 4096->12288 with
                            RMSNorm hd 256; FFN up 3072->2x12288 with SwiGLU and
                            MXFP4 re-quantisation of the output.
  dit_block                 batch of 4 images (16384 tokens): block transform +
                            quantise of every input, QKV (RMSNorm hd 128), FFN up
                            (SwiGLU, bf16 out), FFN down (no epilogue).
  dit_1k_linears_unfused    the DiT-1K linears without epilogue fusion: each GEMM
                            stores bf16, then RMSNorm / SwiGLU run as launches of
                            their own and the SwiGLU output is quantised by the
                            activation quantiser (what the fused epilogues save).
  dit_block_fused           the same block with the down projection's input made
                            in the FFN-up epilogue: SwiGLU -> down transform ->
                            MXFP4, so h never reaches HBM and the down layer has
                            no transform + quantise pass of its own.

Prints one JSON line.  TFLOP/s counts 2*M*N*K per GEMM (N the physical width).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_MXFP4_TFLOPS = 10100.0     # MI355X dense MXFP4 matrix peak
PER_LAYER_STEPS = 20       # untimed steps after the timed ones, for every GEMM's duration
PEAK_CLOCK_GHZ = 2.4            # the clock that peak is quoted at
PEAK_HBM_GBS = 8000.0
QUANT_BATCH = 20               # back-to-back launches timed for the quantisation figure
HBM_ROTATE_BYTES = 512 << 20   # buffer sets rotated by an HBM-bound timing touch more than 2x the LLC
LATENT_SHAPE = (16, 16, 128, 128)   # sampler updates: 16 latents of a 1024x1024 image (16 ch, 8x down)
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--warm-seconds", type=float, default=0.5,
                   help="untimed steps run for this long before the warmup steps: under a sustained FP4 "
                        "MFMA load the GPU's clock settles within tens of milliseconds, and a timed region "
                        "that starts from idle reads 10-15%% slow")
    p.add_argument("--workload", default="dit_1k_linears", choices=["dit_1k_linears", "dit_1k_linears_unfused", "dit_block",
                                                                 "dit_block_fused"])
    p.add_argument("--rotate", type=int, default=4, help="activation buffer copies cycled over steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra-configs", action="store_true",
                   help="skip the tiny and batch-4 block records that follow the headline workload")
    p.add_argument("--extra-steps", type=int, default=30, help="timed steps of each batch-4 block record")
    p.add_argument("--calib-mib", type=int, default=0,
                   help="before warm-up, fill a buffer of this many MiB once and then sum it, so that HBM "
                        "write and read counters can be calibrated against kernels of known traffic")
    return p.parse_args()


# ------------------------------------------------------------------ layers --
class Layer:
    """One fused linear: activations -> [transform +] quantise -> GEMM + epilogue."""

    def __init__(self, name, wl, ops, torch, rotate, x_override=None, transform=None):
        self.name, self.wl = name, wl
        dev = "cuda"
        self.m, self.k = wl.m, wl.k
        x = wl.x if x_override is None else x_override
        xs = [torch.from_numpy(x).to(dev, torch.bfloat16 if wl.x_bf16 else torch.float32)]
        for r in range(1, rotate):                     # distinct copies defeat the LLC
            xs.append(xs[0].clone())
        self.xs = xs
        self.t = None if transform is None else torch.from_numpy(transform).to(dev, torch.bfloat16)
        if wl.epilogue == "swiglu":
            w = np.concatenate([wl.w_gate, wl.w_up], axis=1)
            group = ops.swiglu_interleave_group()
        else:
            w = wl.w
            group = 0
        wd = torch.from_numpy(w).to(dev, torch.float32)
        if self.t is not None:
            wd = ops.fold_inverse_transform(wd, self.t)
        self.b = ops.pack_weight(wd, interleave_group=group)          # tiled MXFP4 [N, K]
        del wd
        self.n = self.b.rows
        self.a = ops.mx_empty(self.m, self.k, "tiled", dev)
        if wl.epilogue == "swiglu":
            self.out = torch.empty((self.m, self.n // 2), dtype=torch.bfloat16, device=dev) \
                if not wl.requant else None
            self.req = ops.mx_empty(self.m, self.n // 2, "tiled", dev) if wl.requant else None
        else:
            self.out = torch.empty((self.m, self.n), dtype=torch.bfloat16, device=dev)
        if wl.epilogue == "rmsnorm_head":
            self.norm_w = torch.from_numpy(wl.norm_w).to(dev, torch.float32)
        self.flops = 2 * self.m * self.n * self.k
        self.ops = ops
        self.next_t = None          # set: SwiGLU -> this block transform -> MXFP4 into next_a
        self.next_a = None
        self.unfused = False

    def make_unfused(self, torch):
        """GEMM with a bf16 store, then the epilogue as launches of its own."""
        self.unfused = True
        self.c = torch.empty((self.m, self.n), dtype=torch.bfloat16, device="cuda")
        if self.wl.epilogue == "swiglu":
            self.h = torch.empty((self.m, self.n // 2), dtype=torch.bfloat16, device="cuda")

    def quantize(self, step):
        if self.xs is None:         # activations made by the previous layer's epilogue
            return
        x = self.xs[step % len(self.xs)]
        if self.t is not None:
            self.ops.block_transform(x, self.t, quantize=True, out=self.a)
        else:
            self.ops.quantize_mxfp4(x, out=self.a)

    def gemm(self):
        ops, wl = self.ops, self.wl
        if self.unfused:
            ops.gemm_fp4_epilogue_none(self.a, self.b, out=self.c)
        elif wl.epilogue == "rmsnorm_head":
            ops.gemm_fp4_epilogue_rmsnorm_head(self.a, self.b, wl.head_dim, wl.n_norm, self.norm_w, wl.eps,
                                               out=self.out)
        elif wl.epilogue == "swiglu" and self.next_t is not None:
            ops.gemm_fp4_epilogue_swiglu_transform(self.a, self.b, self.next_t, out_mx=self.next_a)
        elif wl.epilogue == "swiglu":
            ops.gemm_fp4_epilogue_swiglu(self.a, self.b, out_dtype=None, requant=wl.requant, out=self.out,
                                         out_mx=self.req)
        else:
            ops.gemm_fp4_epilogue_none(self.a, self.b, out=self.out)

    def epilogue(self):
        """The unfused epilogue launches (nothing when the GEMM fuses it)."""
        if not self.unfused:
            return
        ops, wl = self.ops, self.wl
        if wl.epilogue == "rmsnorm_head":
            ops.rmsnorm_head(self.c, wl.head_dim, wl.n_norm, self.norm_w, wl.eps, out=self.out)
        elif wl.epilogue == "swiglu":
            ops.swiglu(self.c, ops.swiglu_interleave_group(), out=self.h)
            if wl.requant:
                ops.quantize_mxfp4(self.h, out=self.req)

    def epilogue_bytes(self):
        """Algorithmic HBM bytes of the unfused epilogue launches."""
        mn = self.m * self.n
        if self.wl.epilogue == "rmsnorm_head":
            return 2 * mn + 2 * mn                          # bf16 C in, bf16 y out
        b = 2 * mn + mn                                     # bf16 C in, bf16 h [M, N/2] out
        if self.wl.requant:
            b += mn + self.m * (self.n // 4 + self.n // 64)   # h in, codes + scales out
        return b

    def quant_bytes(self):
        """Algorithmic HBM bytes of the activation quantiser: bf16 in, codes + scales out."""
        if self.xs is None:
            return 0
        return self.m * self.k * (2 if self.wl.x_bf16 else 4) + self.m * self.k // 2 + self.m * self.k // 32

    def gemm_bytes(self):
        """Algorithmic HBM bytes of the fused GEMM: both MXFP4 operands once, output once."""
        ab = self.m * self.k // 2 + self.m * self.k // 32
        bb = self.n * self.k // 2 + self.n * self.k // 32
        if self.unfused:
            ob = self.m * self.n * 2
        elif self.wl.epilogue == "swiglu":
            ob = self.m * (self.n // 4 + self.n // 64) if (self.wl.requant or self.next_t is not None) \
                else self.m * self.n
        else:
            ob = self.m * self.n * 2
        return ab + bb + ob


def build_layers(args, ops, torch, workloads):
    if args.workload in ("dit_1k_linears", "dit_1k_linears_unfused"):
        wls = [workloads.qkv_hd128(), workloads.qkv_hd256(), workloads.ffn_up_swiglu(requant=True)]
        layers = [Layer(w.name, w, ops, torch, args.rotate) for w in wls]
        if args.workload == "dit_1k_linears_unfused":
            for L in layers:
                L.make_unfused(torch)
        return layers
    qkv, up, down = workloads.dit_block()
    layers = [Layer("dit_block_qkv", qkv, ops, torch, args.rotate, transform=qkv.t),
              Layer("dit_block_up", up, ops, torch, args.rotate, transform=up.t)]
    # The down projection's input is the up projection's bf16 SwiGLU output.
    up_layer = layers[1]
    up_layer.wl.requant = False
    n_half = up_layer.n // 2
    up_layer.out = torch.empty((up_layer.m, n_half), dtype=torch.bfloat16, device="cuda")
    up_layer.req = None
    dl = Layer("dit_block_down", down, ops, torch, 1, transform=down.t)
    if args.workload == "dit_block_fused":
        # The up epilogue writes the down layer's MXFP4 activations directly.
        up_layer.out = None
        up_layer.next_t, up_layer.next_a = dl.t, dl.a
        dl.xs = None
    else:
        dl.xs = [up_layer.out]                                     # chained: the up layer's bf16 output
    layers.append(dl)
    return layers


# --------------------------------------------------------------- measuring --
def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_diffusion_transformer_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, kernel_key):
    """Bytes per launch that leave the L2 (an upper bound on HBM bytes: no
    counter separates Infinity Cache hits) from the committed rocprofv3
    counter summary of this workload, if it was taken on the current kernel
    sources; else None."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel_key)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(args, layers_wl, rows=2048, min_seconds=10.0, max_windows=8):
    """The oracle as it stands, on a bounded sample of the same workload:
    windows of `rows` consecutive tokens of every layer, taken in turn (wrapping
    around the layer's tokens) until at least `min_seconds` of oracle work have
    been timed.  Timed: activation [transform +] quantise, the
    dequantise-then-fp64 GEMM and the epilogue; weight quantisation (offline
    on both sides) is outside the timed region."""
    sys.path.insert(0, ROOT)
    from oracle import gemm as ogemm
    from oracle import mxfp4
    from oracle import transform as otransform
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:  # noqa: BLE001
        threads = 1
    prepared = []
    for wl in layers_wl:
        t = None if wl.t is None else wl.t.astype(np.float64)
        if wl.epilogue == "swiglu":
            wg, wu = wl.w_gate.astype(np.float64), wl.w_up.astype(np.float64)
            if t is not None:
                wg, wu = otransform.fold_inverse(wg, t), otransform.fold_inverse(wu, t)
            gc_, gs_ = mxfp4.quantize(wg.T)
            uc_, us_ = mxfp4.quantize(wu.T)
            bc = bs = None
            n = 2 * wl.w_gate.shape[1]
        else:
            w = wl.w.astype(np.float64)
            if t is not None:
                w = otransform.fold_inverse(w, t)
            bc, bs = mxfp4.quantize(w.T)
            gc_ = gs_ = uc_ = us_ = None
            n = wl.w.shape[1]
        prepared.append((wl, t, n, bc, bs, gc_, gs_, uc_, us_))
    flops, elapsed, windows = 0, 0.0, 0
    while windows < max_windows and (windows == 0 or elapsed < min_seconds):
        for wl, t, n, bc, bs, gc_, gs_, uc_, us_ in prepared:
            r0 = (windows * rows) % max(wl.m - rows + 1, 1)
            x = wl.x[r0:r0 + rows].astype(np.float64)
            t1 = time.perf_counter()
            ac, as_ = mxfp4.quantize(x) if t is None else otransform.transform_quantize(x, t)
            if wl.epilogue == "swiglu":
                h = ogemm.swiglu(ogemm.gemm(ac, as_, gc_, gs_), ogemm.gemm(ac, as_, uc_, us_))
                if wl.requant:
                    ogemm.requantize(h)
            else:
                c = ogemm.gemm(ac, as_, bc, bs)
                if wl.epilogue == "rmsnorm_head":
                    ogemm.rmsnorm_head(c, wl.head_dim, wl.n_norm, wl.norm_w.astype(np.float64), wl.eps)
            elapsed += time.perf_counter() - t1
            flops += 2 * x.shape[0] * n * wl.k
        windows += 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "blas_threads": int(threads), "cpu_count": os.cpu_count(),
            "sched_affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "sample": "%d windows of %d tokens of each layer of the workload (%s); %.1f s timed" % (
                windows, rows, ", ".join(w.name for w in layers_wl), elapsed)}


def time_rotating(torch, launches, n=QUANT_BATCH):
    """Average ms of one launch over n back-to-back launches cycling through
    `launches` (closures over distinct, preallocated buffer sets).  The n
    launches are captured in a HIP graph and timed as one replay, so the
    host's per-call cost (argument checks, ctypes) leaves no gaps between
    these ~10 us kernels."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for f in launches:                                   # untimed pass
        f()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            launches[i % len(launches)]()
    graph.replay()                                       # untimed replay
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def n_sets(bytes_per_set):
    return max(2, -(-HBM_ROTATE_BYTES // bytes_per_set))


def hbm_record(kernel, nbytes, ms, what):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_launch_ms": round(ms, 5), "algorithmic_bytes": nbytes,
            "measured": what}


def aux_kernels(torch, ops, workloads):
    """The next-row kernels, each HBM-bound, timed on rotating buffer sets:
    QAD fake quantisation of a DiT-1K activation and the three sampler updates
    on a batch of latents (fp32)."""
    out = []
    wl = workloads.ffn_up_swiglu()
    x = torch.from_numpy(wl.x).to("cuda", torch.bfloat16)
    nb = x.numel() * 4                                   # bf16 in, bf16 out
    sets = [(x.clone(), torch.empty_like(x)) for _ in range(n_sets(nb))]
    ms = time_rotating(torch, [lambda a=a, b=b: ops.fake_quantize_mxfp4(a, out=b) for a, b in sets])
    out.append(hbm_record("fake_quantize_mxfp4 (QAD forward, %dx%d bf16 -> bf16)" % tuple(x.shape), nb, ms,
                          "%d launches over %d buffer sets, one graph replay" % (QUANT_BATCH, len(sets))))
    del sets
    n = int(np.prod(LATENT_SHAPE))
    g = torch.Generator(device="cuda").manual_seed(0)
    d, c0, c1 = ops.etd_coefficients(0.8, 0.6, 0.9, 0.43589, order=2)
    for name, n_in, fn in (
            ("etd1_update", 2, lambda t: ops.etd1_update(t[0], t[1], d, c0 + c1, out=t[-1])),
            ("etd2_update", 3, lambda t: ops.etd2_update(t[0], t[1], t[2], d, c0, c1, out=t[-1])),
            ("richardson_combine", 2, lambda t: ops.richardson_combine(t[0], t[1], 4.0, out=t[-1]))):
        nb = (n_in + 1) * n * 4
        sets = [[torch.randn(n, device="cuda", generator=g) for _ in range(n_in + 1)] for _ in range(n_sets(nb))]
        ms = time_rotating(torch, [lambda t=t: fn(t) for t in sets])
        out.append(hbm_record("%s (%d latents %s fp32)" % (name, LATENT_SHAPE[0], "x".join(map(str, LATENT_SHAPE[1:]))),
                              nb, ms, "%d launches over %d buffer sets, one graph replay" % (QUANT_BATCH, len(sets))))
        del sets
    return out


def measure_steps(torch, layers, steps, warmup, warm_seconds, per_layer_steps=PER_LAYER_STEPS):
    """ms per step of `layers` (each step: every layer's quantise, GEMM and
    unfused epilogue, if any) over `steps` timed steps after warm-up, and
    every layer's GEMM duration from per_layer_steps more steps with events
    around each GEMM."""
    def step(s, ev=None):
        for i, L in enumerate(layers):
            L.quantize(s)
            if ev is not None:
                ev[(i, 0)][s].record()
            L.gemm()
            if ev is not None:
                ev[(i, 1)][s].record()
            L.epilogue()

    t_warm = time.perf_counter()
    s = 0
    while time.perf_counter() - t_warm < warm_seconds:
        step(s)
        s += 1
        if s % 20 == 0:
            torch.cuda.synchronize()
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(steps):
        step(s)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    ev = {(i, k): [torch.cuda.Event(enable_timing=True) for _ in range(per_layer_steps)]
          for i in range(len(layers)) for k in (0, 1)}
    for s in range(per_layer_steps):
        step(s, ev)
    torch.cuda.synchronize()
    gemms = []
    for i, L in enumerate(layers):
        us = 1e3 * float(np.mean([ev[(i, 0)][s].elapsed_time(ev[(i, 1)][s]) for s in range(per_layer_steps)]))
        tf = L.flops / (us * 1e-6) / 1e12
        gemms.append({"layer": L.name, "M": L.m, "N": L.n, "K": L.k, "avg_us": round(us, 2),
                      "tflops": round(tf, 1), "frac": round(tf / PEAK_MXFP4_TFLOPS, 4)})
    return ms_step, gemms


def transform_record(torch, L):
    """GB/s of the layer's block transform + quantise, over enough input
    copies that every launch reads HBM, as one graph replay."""
    sets = [L.xs[0].clone() for _ in range(n_sets(L.quant_bytes()))]
    saved = L.xs
    L.xs = sets
    ms = time_rotating(torch, [lambda i=i: L.quantize(i) for i in range(len(sets))])
    L.xs = saved
    del sets
    return hbm_record("block_transform + quantise (%s, %dx%d bf16, %d matrices)" % (L.name, L.m, L.k, L.k // 32),
                      L.quant_bytes(), ms, "%d launches over %d input copies, one graph replay"
                      % (QUANT_BATCH, n_sets(L.quant_bytes())))


def block_record(ms_step, layers, gemms, workload):
    flops = sum(L.flops for L in layers)
    tf = flops / (ms_step * 1e-3) / 1e12
    return {"workload": workload, "ms_per_step": round(ms_step, 5), "tflops": round(tf, 2),
            "pct_of_mxfp4_peak": round(100.0 * tf / PEAK_MXFP4_TFLOPS, 2),
            "layers": [{"name": L.name, "M": L.m, "N": L.n, "K": L.k,
                        "input": "block transform + quantise" if L.xs is not None
                        else "MXFP4 from the previous layer's epilogue",
                        "epilogue": L.wl.epilogue + ("+down_transform+requant" if L.next_t is not None else "")}
                       for L in layers],
            "gemms": gemms}


def extra_configs(args, torch, ops, workloads):
    """The other configurations, timed in the same run after the headline:
    the tiny 256x512x512 case (latency; launch-bound) and the batch-4 DiT
    block (16384 tokens, block transform on every input), unfused and with
    the FFN-up epilogue producing the down projection's MXFP4 input."""
    out = {}
    # tiny: fp32 X [256, 512] -> quantise -> GEMM + RMSNorm hd 128 (4 heads)
    wl = workloads.tiny()
    L = Layer("tiny", wl, ops, torch, 1)

    def tiny_step(s=0):
        L.quantize(0)
        L.gemm()

    for _ in range(50):
        tiny_step()
    torch.cuda.synchronize()
    n = 200
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        tiny_step()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            tiny_step()
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / n
    out["tiny"] = {"workload": "tiny: X fp32 [256, 512] -> MXFP4 -> GEMM 256x512x512 + RMSNorm hd 128 (4 heads), "
                               "bf16 out", "us_per_step_eager": round(eager_us, 2),
                   "us_per_step_graph": round(graph_us, 2),
                   "tflops_graph": round(L.flops / (graph_us * 1e-6) / 1e12, 2),
                   "measured": "%d back-to-back steps (quantise + GEMM), events around them; eager launches, "
                               "then the same steps as one HIP-graph replay" % n,
                   "bound": "launch / latency (0.134 GFLOP)"}
    del L, graph
    # the batch-4 block, unfused then fused; the weights are prepared once
    bargs = argparse.Namespace(**vars(args))
    bargs.workload = "dit_block"
    layers = build_layers(bargs, ops, torch, workloads)
    ms, gemms = measure_steps(torch, layers, args.extra_steps, 5, 0.3)
    rec = block_record(ms, layers, gemms, "dit_block")
    rec["block_transform"] = transform_record(torch, layers[2])
    out["dit_block"] = rec
    up, dl = layers[1], layers[2]
    up.out, up.next_t, up.next_a = None, dl.t, dl.a
    dl.xs = None
    ms, gemms = measure_steps(torch, layers, args.extra_steps, 5, 0.3)
    out["dit_block_fused"] = block_record(ms, layers, gemms, "dit_block_fused")
    del layers
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the path runs on one GPU; --gpus %d is not supported "
              "(the path shards by tokens with no exchange between GPUs)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, ROOT)
    from fp4_diffusion_transformer_amd import clockprobe, ops, workloads

    torch.cuda.init()
    clk_idle = clockprobe.shader_clock_ghz(1, 64)   # one workgroup, before any load (the shader-clock probe)
    if args.calib_mib:
        buf = torch.empty(args.calib_mib << 18, dtype=torch.float32, device="cuda")
        buf.fill_(1.0)                       # writes calib_mib MiB
        torch.cuda.synchronize()
        total = buf.sum()                    # reads calib_mib MiB
        torch.cuda.synchronize()
        del buf, total
    layers = build_layers(args, ops, torch, workloads)
    torch.cuda.synchronize()

    # dominant kernel = the GEMM with the most flops in a step
    dom = max(range(len(layers)), key=lambda i: layers[i].flops)
    quant_dom = max(range(len(layers)), key=lambda i: layers[i].quant_bytes())

    def step(s, ev=None, bracket=None):
        # ev: events around the GEMMs of the layers in `bracket` (default: the dominant one)
        for i, L in enumerate(layers):
            L.quantize(s)
            timed = ev is not None and i in (bracket or (dom,))
            if timed:
                ev[(i, 0)][s].record()
            L.gemm()
            if timed:
                ev[(i, 1)][s].record()
            L.epilogue()

    t_warm = time.perf_counter()
    s = 0
    while time.perf_counter() - t_warm < args.warm_seconds:
        step(s)
        s += 1
        if s % 20 == 0:
            torch.cuda.synchronize()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    ev = {(dom, k): [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] for k in (0, 1)}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(s, ev)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Every layer's GEMM duration, from PER_LAYER_STEPS more steps of the same
    # mix with events around all of its GEMMs.  Kept out of the timed steps:
    # each event record puts a few microseconds between kernels (four more
    # per step cost the step 3.5%).
    all_layers = tuple(range(len(layers)))
    ev_all = {(i, k): [torch.cuda.Event(enable_timing=True) for _ in range(PER_LAYER_STEPS)]
              for i in all_layers for k in (0, 1)}
    for s in range(PER_LAYER_STEPS):
        step(s, ev_all, all_layers)
    torch.cuda.synchronize()
    # the clock under a sustained FP4 MFMA load: right after the timed region,
    # the probe loads every CU with FP4 MFMAs for about a millisecond (the
    # steps' own clock, read inside the GEMM the same way in a timing copy,
    # agrees within a few per cent); its MFMA rate is the box's practical
    # matrix ceiling at that clock
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    probe = torch.zeros(12 * cus, dtype=torch.int64, device="cuda")
    p_iters = 3000
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record()
    clockprobe.clock_probe(probe, cus, p_iters)
    pe1.record()
    torch.cuda.synchronize()
    clk_load = float(np.median(clockprobe.clock_ghz(probe, cus)))
    mfma_pf = 2.0 * 32 * 32 * 64 * 16 * p_iters * 4 * cus / (pe0.elapsed_time(pe1) * 1e-3) / 1e15
    del probe
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    flops = sum(L.flops for L in layers)
    tflops = flops / (ms_step * 1e-3) / 1e12

    g_ms = [ev[(dom, 0)][s].elapsed_time(ev[(dom, 1)][s]) for s in range(args.steps)]
    per_gemm = []
    for i, L in enumerate(layers):
        us = 1e3 * float(np.mean([ev_all[(i, 0)][s].elapsed_time(ev_all[(i, 1)][s])
                                  for s in range(PER_LAYER_STEPS)]))
        tf = L.flops / (us * 1e-6) / 1e12
        per_gemm.append({"layer": L.name, "M": L.m, "N": L.n, "K": L.k, "avg_us": round(us, 2),
                         "tflops": round(tf, 1), "frac": round(tf / PEAK_MXFP4_TFLOPS, 4)})
    g_avg = float(np.mean(g_ms))
    # The activation-quantisation kernel is ~10 us: a pair of events around a
    # single launch would mostly time the dispatch gap, so after the timed
    # region it is timed over QUANT_BATCH back-to-back launches instead, on
    # enough input copies that no launch reads what the last-level cache holds.
    Lq = layers[quant_dom]
    q_sets = [Lq.xs[0].clone() for _ in range(n_sets(Lq.quant_bytes()))]
    saved = Lq.xs
    Lq.xs = q_sets
    q_avg = time_rotating(torch, [lambda i=i: Lq.quantize(i) for i in range(len(q_sets))])
    Lq.xs = saved
    del q_sets
    Ld = layers[dom]
    achieved = Ld.flops / (g_avg * 1e-3) / 1e12
    # kernel instantiation as rocprof names it: epilogue, bf16 output, LDS ring
    # depth (3) and the K stages peeled before its unrolled loop
    # output kind template argument: 0 no `out` (requant only), 1 bf16, 2 fp32
    out_kind = 1 if (Ld.out is not None or Ld.unfused) else 0
    kt, ring = Ld.k // 128, 3
    epi_name = "none" if Ld.unfused else Ld.wl.epilogue + ("_transform" if Ld.next_t is not None else "")
    peel = (kt - ring + 1) % ring                  # as the library picks it: a whole ring turn
    if peel == 0 and kt - ring + 1 >= ring:        # rather than none when the loop would start at 0
        peel = ring
    kernel_key = "gemm_%s<%d,%d,%d>" % (epi_name, out_kind, ring, peel)

    out = {
        "metric": "fused MXFP4 GEMM+epilogue TFLOPS and % of MXFP4 peak at DiT 1K shapes",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "layers": [{"name": L.name, "M": L.m, "N": L.n, "K": L.k, "epilogue": L.wl.epilogue
                        + ("+requant" if L.wl.requant else "") + (" (unfused)" if L.unfused else "")
                        + ("+next_transform+requant" if L.next_t is not None else ""),
                        "input": "block transform + quantise" if L.t is not None and L.xs is not None
                        else ("from the previous epilogue" if L.xs is None else "quantise")}
                       for L in layers],
            "pct_of_mxfp4_peak": round(100.0 * tflops / PEAK_MXFP4_TFLOPS, 2),
            "wall_s_timed": round(wall, 3),
        },
        "clock": {
            "method": "shader-clock probe: s_memtime against the 100 MHz s_memrealtime around FP4 MFMAs "
                      "(32x32x64, pseudo-random operands); idle: one workgroup before any work; under load: "
                      "one workgroup per CU for about 1 ms right after the timed region, median over waves",
            "shader_ghz_idle": round(clk_idle, 3),
            "shader_ghz_fp4_mfma_load": round(clk_load, 3),
            "published_max_ghz": PEAK_CLOCK_GHZ,
            "mfma_only_pflops_at_that_clock": round(mfma_pf, 3),
            "pct_of_mxfp4_peak_at_measured_clock": round(
                100.0 * tflops / (PEAK_MXFP4_TFLOPS * clk_load / PEAK_CLOCK_GHZ), 2),
            "dominant_gemm_pct_of_mfma_only_rate": round(100.0 * achieved / (mfma_pf * 1e3), 2),
        },
        "roofline": {
            "kernel": kernel_key + " (%s, M=%d N=%d K=%d)" % (Ld.name, Ld.m, Ld.n, Ld.k),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_MXFP4_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MXFP4_TFLOPS, 4),
            "traffic": traffic_from_profile(args.workload, kernel_key),
            "avg_launch_ms": round(g_avg, 5),
            "algorithmic_bytes": Ld.gemm_bytes(),
        },
        "gemms": per_gemm,
        "quantize_roofline": {
            "kernel": ("block_transform" if Lq.t is not None else "quantize_mxfp4") + " (%s, %dx%d bf16)"
                      % (Lq.name, Lq.m, Lq.k),
            "bound": "hbm",
            "achieved": round(Lq.quant_bytes() / (q_avg * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(Lq.quant_bytes() / (q_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "avg_launch_ms": round(q_avg, 5),
            "measured": "events around one graph replay of %d back-to-back launches after the timed region, "
                        "over %d input copies" % (QUANT_BATCH, n_sets(Lq.quant_bytes())),
            "algorithmic_bytes": Lq.quant_bytes(),
        },
        "aux_kernels": aux_kernels(torch, ops, workloads),
    }
    if any(L.unfused for L in layers):
        # each layer's separate epilogue launches, timed like the quantiser
        epis = []
        for L in layers:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(QUANT_BATCH):
                L.epilogue()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / QUANT_BATCH
            epis.append({"layer": L.name, "avg_ms": round(ms, 5), "bound": "hbm",
                         "achieved_GBs": round(L.epilogue_bytes() / (ms * 1e-3) / 1e9, 1),
                         "algorithmic_bytes": L.epilogue_bytes()})
        out["unfused_epilogues"] = epis
    layer_wls = [L.wl for L in layers]
    if args.workload == "dit_1k_linears" and not args.no_extra_configs:
        del layers, Lq, Ld
        torch.cuda.empty_cache()
        out["configs"] = extra_configs(args, torch, ops, workloads)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, layer_wls)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
