#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE forward (route -> permute -> expert
FFN over low-bit weights -> combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the GLM-5-class decode layer -- 256 experts, top-8,
hidden 6144, expert intermediate 2048, NVFP4 weights quantized from
N(0, 0.02) fp32 -- at a batch of 32 bf16 tokens with uniform-random router
logits.  A step is one whole forward over one batch; the batches rotate over
a pool of seeded inputs resident in HBM (so consecutive steps route to
different experts and the weights stream from HBM, not from the caches).

Prints ONE JSON line on stdout (progress goes to stderr):
  value          tokens/s of the whole path
  roofline       the NVFP4 gate/up kernel: packed gate/up bytes of the
                 experts it touches per launch / its mean launch time
                 (HIP events on the launch stream), against 8 TB/s HBM
  cpu_baseline   the fp64 oracle on a bounded sample (three tokens), one core
  extra          the same path on the other workloads (decode T = 1 and 8,
                 prefill T = 4096 with Zipf(1.1) routing, 2-bit VQ T = 8,
                 small-codebook VQ at 1 and 2 bits per weight T = 8,
                 mixed NVFP4/VQ T = 8 and 32, the same mixed layer with
                 its hot experts switched to the NVFP4 tier at run time,
                 the decode and prefill layers with a BF16 shared expert, and
                 the decode layer stored rotated (online Hadamard-128
                 rotations around every matrix))
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# sources of the decode gate/up kernel (the roofline kernel)
ROOFLINE_SOURCES = ("dev_common.h", "ffn_decode.hip", "internal.h")


# decode batches (T below this) take the weight-streaming kernels, larger ones
# the grouped GEMM
PREFILL_MIN_TOKENS = 128


def gateup_kernel_name(T, k, n_experts):
    """The NVFP4 gate/up decode kernel the library launches for a batch of T
    tokens: its inputs are split over 4 / 2 / 1 waves when at most 16 / 64 /
    more experts can be active (min(T k, experts of the format))."""
    slots = min(T * k, n_experts)
    ks = 4 if slots <= 16 else 2 if slots <= 64 else 1
    return f"k_ffn<NvFmt, 1, {ks}, 2, 0, 4, false, false, false, false>"


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_moe_route_amd", "csrc")
    for f in ROOFLINE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(name):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


# --------------------------------------------------------------------------

class Runner:
    """Pre-allocated buffers and a pool of input batches for one workload."""

    def __init__(self, layer, wl, T, reps, dev, shared=None):
        import numpy as np
        import torch
        import bit_quantized_moe_route_amd as moeq
        import synth

        self.moeq, self.torch = moeq, torch
        self.layer, self.wl, self.T, self.k = layer, wl, T, wl.k
        self.batches = []
        self.touched = []
        for r in range(reps):
            lg = synth.logits(wl, T, rep=r)
            x = synth.activations(wl, T, rep=r)
            self.batches.append((torch.from_numpy(lg).to(dev),
                                 torch.from_numpy(x.view(np.int16)).to(dev)))
            # experts touched (for byte accounting only)
            top = np.argsort(-lg, axis=1, kind="stable")[:, :wl.k]
            self.touched.append(np.unique(top))
        k, E, H, I = wl.k, wl.E, wl.H, wl.I
        i32, f32 = torch.int32, torch.float32
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.perm = (torch.empty(E, dtype=i32, device=dev), torch.empty(E + 1, dtype=i32, device=dev),
                     torch.empty(T * k, dtype=i32, device=dev), torch.empty(T * k, dtype=i32, device=dev))
        self.h = torch.empty((T * k, I), dtype=torch.float16, device=dev)
        self.y = torch.empty((T * k, H), dtype=f32, device=dev)
        self.out = torch.empty((T, H), dtype=f32, device=dev)
        self.ws = moeq.gateup_workspace(layer, T, k)
        self.pws = moeq.permute_workspace(T, k, E, dev)
        self.lws = moeq.layer_workspace(layer, T, k, shared=shared)
        self.shared = shared
        if shared is not None:
            self.y_sh = torch.empty((T, H), dtype=f32, device=dev)
            self.sws = moeq.shared_workspace(shared, T)
        self.ev = []
        self.ev_sh = []

    def step(self, r, timed):
        """One layer forward on batch r.  Untimed (warm-up and the graph
        replays that give the headline figures): the one-call layer,
        moe_layer_forward, or moe_layer_forward_shared with a shared expert
        (fused for decode batches of <= 16 assignments).
        Timed eager steps: the step-by-step calls, with HIP events around the
        gate/up call (the kernel-level figures)."""
        moeq = self.moeq
        lg, x = self.batches[r % len(self.batches)]
        if not timed:
            moeq.layer_forward(self.layer, x, lg, self.k, out=self.out, ids=self.ids, w=self.w,
                               ws=self.lws, shared=self.shared)
            return
        moeq.route_permute(lg, self.k, self.wl.E, (self.ids, self.w) + self.perm, self.pws)
        counts, offsets, perm_src, inv_perm = self.perm
        # the C call with its arguments marshalled before the first event, so
        # the events bracket the kernel rather than Python's overhead
        import ctypes
        L = moeq.lib()
        args = (ctypes.byref(self.layer.c()), moeq._dptr(x), moeq._dptr(perm_src),
                moeq._dptr(offsets), self.T, self.k, moeq._dptr(self.h), moeq._dptr(self.ws),
                self.ws.numel(), moeq._stream(x.device))
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.moe_expert_gateup_q(*args)
        e1.record()
        moeq._check(rc, "moe_expert_gateup_q")
        self.ev.append((r, e0, e1))
        moeq.expert_down_q(self.layer, self.h, offsets, self.k, self.y)
        if self.shared is None:
            moeq.combine(self.y, inv_perm, self.w, self.out)
            return
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        moeq.shared_ffn(self.shared, x, self.y_sh, self.sws)
        e1.record()
        self.ev_sh.append((r, e0, e1))
        moeq.combine_shared(self.y, inv_perm, self.w, self.y_sh, self.out)

    def run(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i, False)
        torch.cuda.synchronize()
        self.ev = []
        self.ev_sh = []
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i, True)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        gu_ms = [e0.elapsed_time(e1) for _, e0, e1 in self.ev]
        return dt, gu_ms

    def run_graph(self, steps, warmup):
        """The same steps replayed from HIP graphs, as a decode loop would run
        them: each graph holds `group` consecutive steps (each on its own input
        batch; group = the largest divisor of `steps` up to 16), so the host's
        per-graph launch cost is paid once per group.  The graphs together
        cover the batch pool a whole number of times.  Returns (seconds, group)."""
        import math
        torch = self.torch
        nb = len(self.batches)
        group = max(d for d in range(1, min(16, steps) + 1) if steps % d == 0)
        ng = nb // math.gcd(group, nb)
        graphs = []
        for gi in range(ng):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for u in range(group):
                    self.step(gi * group + u, False)
            graphs.append(g)
        for i in range(max(1, (warmup + group - 1) // group)):
            graphs[i % ng].replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps // group + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps // group):
            graphs[i % ng].replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        # per-step time of each replay (HIP events between replays)
        self.replay_step_ms = [ev[i].elapsed_time(ev[i + 1]) / group
                               for i in range(steps // group)]
        return dt, group

    def bytes_of(self, r, which):
        """Algorithmic packed-weight bytes of batch r: 'all' (codes + scales
        of every touched expert, VQ codebooks once) or 'gateup'."""
        experts = self.touched[r % len(self.touched)]
        if which == "all":
            sh = self.shared.packed_bytes([0]) if self.shared is not None else 0
            return self.layer.packed_bytes(experts) + sh
        H, I = self.wl.H, self.wl.I
        tot = 0
        for e in experts:
            if self.layer.fmt_host[e] in (self.moeq.FMT_NVFP4, self.moeq.FMT_NVFP4R):
                planes = 2 if self.layer.fmt_host[e] == self.moeq.FMT_NVFP4R else 1
                tot += planes * 2 * (H * I // 2 + H * I // 16)
            elif self.layer.fmt_host[e] == self.moeq.FMT_VQ8:
                tot += 2 * (H * I // 8) * self.layer.vq8_m + 2 * I * 2
            else:
                tot += 2 * (H * I // 8) * 2 + 2 * I * 2
        return tot


def measure(layer, wl, T, steps, warmup, dev, reps=16, shared=None):
    """Eager launches (per-launch HIP events around the gate/up call), then
    the same steps replayed from HIP graphs; the headline figures are the
    graph replay's, the kernel-level ones the eager run's.  A shared expert
    runs after the routed experts on the same stream (its HIP events bracket
    its three launches)."""
    rn = Runner(layer, wl, T, reps, dev, shared)
    dte, gu_ms = rn.run(steps, warmup)
    dt, group = rn.run_graph(steps, warmup)
    idx = list(range(steps))                    # batches of the timed graph replays
    idx_e = [warmup + i for i in range(steps)]  # batches of the timed eager steps
    all_bytes = sum(rn.bytes_of(r, "all") for r in idx)
    gu_bytes = sum(rn.bytes_of(r, "gateup") for r in idx_e)
    gu_s = sum(gu_ms) / 1e3
    import numpy as np
    q = np.percentile(rn.replay_step_ms, [10, 50, 90])
    res = {
        "T": T,
        "tokens_per_s": T * steps / dt,
        "ms_per_step": dt / steps * 1e3,
        "step_ms_p10_p50_p90": [float(v) for v in q],
        "tokens_per_s_eager": T * steps / dte,
        "ms_per_step_eager": dte / steps * 1e3,
        "steps_per_graph": group,
        "packed_GBps": all_bytes / dt / 1e9,
        "packed_frac_hbm": all_bytes / dt / 1e9 / HBM_PEAK_GBS,
        "experts_touched_mean": sum(len(rn.touched[r % reps]) for r in idx) / steps,
        "gateup_ms_mean": sum(gu_ms) / len(gu_ms),
        "gateup_GBps": gu_bytes / gu_s / 1e9,
        "gateup_bytes_per_launch": gu_bytes / steps,
    }
    if shared is not None:
        sh_ms = [e0.elapsed_time(e1) for _, e0, e1 in rn.ev_sh]
        sh_bytes = shared.packed_bytes([0])
        res["shared_ms_mean"] = sum(sh_ms) / len(sh_ms)
        res["shared_GBps"] = sh_bytes / (res["shared_ms_mean"] / 1e3) / 1e9
        res["shared_bytes"] = sh_bytes
    if T >= 1024:
        flops = 6.0 * wl.H * wl.I * T * (wl.k + (1 if shared is not None else 0))
        res["TFLOPs"] = flops / (dt / steps) / 1e12
        res["frac_mfma"] = res["TFLOPs"] / MFMA_F16_PEAK_TFLOPS
        if shared is not None:
            res["shared_TFLOPs"] = 6.0 * wl.H * wl.I * T / (res["shared_ms_mean"] / 1e3) / 1e12
    return res


# --------------------------------------------------------------------------

CPU_SAMPLE_TOKENS = 3


def cpu_baseline(wl, T):
    """The fp64 oracle on the first CPU_SAMPLE_TOKENS tokens of the batch, on
    one core (BLAS threads pinned to 1).  The oracle's own encoder prepares
    the canonical NVFP4 bytes of those tokens' experts in a process pool
    outside the timed region; the timed region is oracle.forward: route,
    decode of the touched experts from canonical bytes, FFN and combine."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    nt = CPU_SAMPLE_TOKENS
    lg = synth.logits(wl, T, rep=0)[:nt]
    x = synth.activations(wl, T, rep=0)[:nt]
    ids, _ = oracle.route_topk(lg, wl.k)
    experts = sorted(int(e) for e in np.unique(ids))
    jobs = [(e, p) for e in experts for p in range(3)]
    ncpu = len(os.sched_getaffinity(0))
    with ProcessPoolExecutor(max(1, min(16, ncpu)), mp_context=mp.get_context("spawn")) as ex:
        enc = list(ex.map(_oracle_encode, [(wl.name, e, p) for e, p in jobs]))
    canon = {}
    for (e, p), cs in zip(jobs, enc):
        canon.setdefault(e, [None, None, None])[p] = cs

    def weights(e):
        return tuple(oracle.nvfp4_dequant(*canon[e][p]) for p in range(3))

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.forward(x, lg, wl.k, weights)
        dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": nt / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"{nt} tokens of the decode T={T} batch ({len(experts)} experts): "
                       f"oracle.forward (fp64 route, NVFP4 decode from canonical bytes, FFN, "
                       f"combine) on one core of '{cpu_model}' ({ncpu} host cores visible); "
                       f"{dt:.1f} s"),
            "seconds": dt}


def _oracle_encode(args):
    import oracle
    import synth
    name, e, p = args
    wl = synth.WORKLOADS[name]
    return oracle.nvfp4_quantize(synth.nvfp4_source_weights(wl, e, p))


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=32, help="decode batch of the headline")
    ap.add_argument("--extra",
                    default="decode1,decode8,prefill,vq,vqprefill,vq1,vq2x8,vq3x8,vq2x8prefill,"
                            "mixed8,mixed32,mixedhot8,"
                            "mixedhot32,nested8,nested32,shared1,shared8,shared32,prefillshared,"
                            "rot1,rot8,rot32,"
                            "rotprefill",
                    help="comma list of other workloads to measure ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if not 1 <= args.T < PREFILL_MIN_TOKENS:
        print(f"--T is the decode batch of the headline: 1 <= T < {PREFILL_MIN_TOKENS} "
              "(prefill sizes are the 'prefill' extra line)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_moe_route_amd as moeq
    import synth
    from bit_quantized_moe_route_amd.layers import build_layer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moeq.lib()
    copy_gbs = None
    if args.probe_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        copy_gbs = 3 * 2 * n / (time.perf_counter() - t0) / 1e9
        log(f"plain 1 GiB copy: {copy_gbs:.0f} GB/s (read + write)")
        del src, dst
    # the HBM read rate the weight-streaming kernels' kind of load reaches on
    # this box (a 4 GiB buffer, read once per launch)
    probe = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = moeq.probe_read(probe)
    for _ in range(2):
        moeq.probe_read(probe, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        moeq.probe_read(probe, sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * probe.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    log(f"HBM read probe (moe_probe_read, 4 GiB): {read_gbs:.0f} GB/s")
    del probe, sink
    wl = synth.DECODE
    t0 = time.perf_counter()
    log("building the NVFP4 decode layer (256 experts, H 6144, I 2048) ...")
    nv_layer = build_layer(wl.E, wl.H, wl.I, synth.tier_map(wl),
                           nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wl, e, p),
                           device=dev, workers=16)
    log(f"  built in {time.perf_counter() - t0:.1f} s")

    log(f"headline: decode T={args.T}, {args.steps} steps after {args.warmup} warm-up")
    head = measure(nv_layer, wl, args.T, args.steps, args.warmup, dev)
    log("  ", json.dumps(head))

    extra = {}
    wanted = [s for s in args.extra.split(",") if s]
    layers = {}
    for name in wanted:
        try:
            if name.startswith("shared") or name == "prefillshared":
                # the NVFP4 layer (same routed experts, routing and tokens) with
                # a BF16 shared expert of intermediate size I
                ws_ = synth.PREFILL_SHARED if name == "prefillshared" else synth.DECODE_SHARED
                if "shared" not in layers:
                    log("building the BF16 shared expert ...")
                    layers["shared"] = build_layer(
                        1, ws_.H, ws_.I, np.array([moeq.FMT_BF16], np.uint8),
                        bf16_weights=lambda e, p: synth.shared_weights_bf16(synth.DECODE_SHARED, p),
                        device=dev, workers=1)
                if name == "prefillshared":
                    extra[name] = measure(nv_layer, ws_, 4096, 5, 2, dev, reps=4,
                                          shared=layers["shared"])
                else:
                    T = int(name[len("shared"):])
                    extra[name] = measure(nv_layer, ws_, T, 30, 5, dev, shared=layers["shared"])
            elif name.startswith("rot"):
                # the same NVFP4 codes read as the rotated matrices of a rotated
                # layer: the decode layer with each expert's signs attached
                wr = synth.DECODE_ROT
                nv_layer.set_rot_signs(np.stack([
                    moeq.pack_rot_signs(*[synth.rot_signs(wr, e, sd) for sd in range(5)],
                                        wr.H, wr.I) for e in range(wr.E)]))
                try:
                    if name == "rotprefill":
                        wpr = synth.Workload("prefill_rot", 2, 256, 8, 6144, 2048, (4096,),
                                             "nvfp4", "zipf", zipf_s=1.1, rot=True)
                        extra[name] = measure(nv_layer, wpr, 4096, 5, 2, dev, reps=4)
                    else:
                        extra[name] = measure(nv_layer, wr, int(name[len("rot"):]), 30, 5, dev)
                finally:
                    nv_layer.set_rot_signs(None)
            elif name.startswith("decode"):
                T = int(name[len("decode"):])
                extra[name] = measure(nv_layer, wl, T, 30, 5, dev)
            elif name == "prefill":
                extra[name] = measure(nv_layer, synth.PREFILL, 4096, 5, 2, dev, reps=4)
            elif name in ("vq", "vqprefill"):
                wq = synth.VQ
                if "vq" not in layers:
                    log("building the VQ layer ...")
                    layers["vq"] = build_layer(
                        wq.E, wq.H, wq.I, synth.tier_map(wq),
                        vq_codes=lambda e, p: (synth.vq_codes(wq, e, p),
                                               synth.vq_scales(wq, e, p)),
                        codebooks=[synth.vq_codebook(wq, p) for p in range(3)], device=dev,
                        workers=16)
                if name == "vqprefill":
                    wp = synth.Workload(name, 2, wq.E, wq.k, wq.H, wq.I, (4096,), "vq", "zipf",
                                        zipf_s=1.1, vq_cfg=wq.vq_cfg)
                    extra[name] = measure(layers["vq"], wp, 4096, 3, 1, dev, reps=4)
                else:
                    extra[name] = measure(layers["vq"], wq, 8, 30, 5, dev)
            elif name in ("vq1", "vq2x8", "vq3x8", "vq1prefill", "vq2x8prefill", "vq3x8prefill"):
                w8 = synth.WORKLOADS[name.replace("prefill", "")]
                log(f"building the small-codebook VQ layer {name} ...")
                lay8 = build_layer(
                    w8.E, w8.H, w8.I, synth.tier_map(w8),
                    vq8_codes=lambda e, p: (synth.vq8_codes(w8, e, p), synth.vq_scales(w8, e, p)),
                    codebooks8=[synth.vq8_codebooks(w8, p) for p in range(3)], vq8_m=w8.vq8_m,
                    device=dev, workers=16)
                if name.endswith("prefill"):
                    # the same layer at T = 4096 with the prefill routing
                    wp = synth.Workload(name, 2, w8.E, w8.k, w8.H, w8.I, (4096,), "vq8", "zipf",
                                        zipf_s=1.1, vq_cfg=w8.vq_cfg, vq8_m=w8.vq8_m)
                    extra[name] = measure(lay8, wp, 4096, 3, 1, dev, reps=4)
                else:
                    extra[name] = measure(lay8, w8, 8, 30, 5, dev)
                del lay8
            elif name.startswith("nested"):
                # the decode layer's experts held nested: two-level records
                # resident, the hot experts lifted to the two-level tier, the
                # rest on the records' base planes
                wn = synth.NESTED
                T = int(name[len("nested"):])
                if "nested" not in layers:
                    log("building the nested two-level NVFP4 layer ...")
                    layers["nested"] = build_layer(
                        wn.E, wn.H, wn.I, synth.tier_map(wn),
                        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wn, e, p),
                        device=dev, workers=16,
                        resident_formats={moeq.FMT_NVFP4, moeq.FMT_NVFP4R},
                        nvfp4r_shift=synth.NVFP4R_SHIFT)
                extra[name] = measure(layers["nested"], wn, T, 30, 5, dev)
            elif name.startswith("mixedhot"):
                # the mixed layer packed in both formats (resident), its tier map
                # switched at run time so that the hot experts take the 4-bit tier
                wm = synth.MIXED
                T = int(name[len("mixedhot"):])
                if "mixed_resident" not in layers:
                    layers.pop("mixed", None)
                    log("building the mixed layer with both formats resident ...")
                    layers["mixed_resident"] = build_layer(
                        wm.E, wm.H, wm.I, synth.tier_map(wm),
                        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wm, e, p),
                        vq_codes=lambda e, p: (synth.vq_codes(wm, e, p), synth.vq_scales(wm, e, p)),
                        codebooks=[synth.vq_codebook(wm, p) for p in range(3)], device=dev,
                        workers=16, resident_formats={moeq.FMT_NVFP4, moeq.FMT_VQ})
                    layers["mixed_resident"].set_tiers(synth.tier_map_hot(wm))
                extra[name] = measure(layers["mixed_resident"], wm, T, 30, 5, dev)
            elif name.startswith("mixed"):
                wm = synth.MIXED
                T = int(name[len("mixed"):])
                if "mixed" not in layers:
                    log("building the mixed layer ...")
                    layers["mixed"] = build_layer(
                        wm.E, wm.H, wm.I, synth.tier_map(wm),
                        nvfp4_weights=lambda e, p: synth.nvfp4_source_weights(wm, e, p),
                        vq_codes=lambda e, p: (synth.vq_codes(wm, e, p), synth.vq_scales(wm, e, p)),
                        codebooks=[synth.vq_codebook(wm, p) for p in range(3)], device=dev,
                        workers=16)
                extra[name] = measure(layers["mixed"], wm, T, 30, 5, dev)
            log(f"  {name}:", json.dumps(extra[name]))
        except Exception as exc:  # report, keep the headline
            extra[name] = {"error": repr(exc)}
            log(f"  {name} failed: {exc!r}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the oracle on a {CPU_SAMPLE_TOKENS}-token sample ...")
        cpu = cpu_baseline(wl, args.T)
        cpu.pop("seconds", None)
        log("  ", json.dumps(cpu))

    achieved = head["gateup_GBps"]
    traffic = read_traffic(f"traffic_gateup_nvfp4_decode_T{args.T}.json")
    line = {
        "metric": "routed-expert tokens/s + packed-weight HBM GB/s (decode M=1..32, prefill 4K)",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights (e2m1+e4m3), fp16 MFMA operands, fp32 accumulate/outputs",
        "data": "synthetic (seeded), resident in HBM",
        "config": {"workload": f"decode layer: 256 experts, top-8, H 6144, I 2048, NVFP4, "
                               f"T={args.T} bf16 tokens, uniform router logits",
                   "experts_touched_mean": head["experts_touched_mean"],
                   "parallelism": "1 GPU"},
        "packed_GBps": head["packed_GBps"],
        "hbm_read_probe_GBps": read_gbs,
        "roofline": {"bound": "hbm",
                     "kernel": gateup_kernel_name(args.T, wl.k, wl.E) + " (NVFP4 gate/up + SwiGLU)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": head["gateup_bytes_per_launch"],
                     "launch_ms_mean": head["gateup_ms_mean"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
