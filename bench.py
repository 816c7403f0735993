#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE forward (route -> permute -> expert
FFN over low-bit weights -> combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--detail-out PATH]

Headline workload: the GLM-5-class decode layer -- 256 experts, top-8,
hidden 6144, expert intermediate 2048, NVFP4 weights quantized from
N(0, 0.02) fp32 -- at a batch of 32 bf16 tokens with uniform-random router
logits.  A step is one whole forward over one batch; the batches rotate over
a pool of seeded inputs resident in HBM (so consecutive steps route to
different experts and the weights stream from HBM, not from the caches).

Prints ONE compact JSON line on stdout (progress goes to stderr):
  value            tokens/s of the whole path (graph replays)
  roofline         the dominant kernel, the NVFP4 gate/up decode kernel:
                   packed gate/up bytes of the experts it touches per launch
                   / its mean launch time (HIP events on the launch stream),
                   against 8 TB/s HBM
  roofline_ffn     the expert FFN of the headline step: all packed bytes of
                   the touched experts / the time of its FFN kernels (gate/up
                   + down), against 8 TB/s
  roofline_prefill the grouped GEMM of the prefill workload (T = 4096,
                   Zipf(1.1) routing): 6 H I T k flop / the time of its
                   gate/up + down kernels, against 2.5 PFLOP/s fp16 MFMA
  cpu_baseline     the fp64 oracle on a bounded sample of the headline batch,
                   a process pool over experts on the host's cores
  extra            per workload: T, tokens/s, ms per step, the bound, and
                   the fraction of that roofline reached by its FFN kernels
                   (decode T = 1 and 8, prefill, 2-bit VQ, small-codebook VQ,
                   mixed NVFP4/VQ, the mixed layer with its hot experts on the
                   NVFP4 tier, nested two-level NVFP4, a BF16 shared expert,
                   rotated layers)
--detail-out writes every figure of every workload to a JSON file.
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

# device clock cycles, per timed step, of the spin kernel queued ahead of the
# eager timed steps (about 0.4 ms at 2.4 GHz: longer than the host takes to
# issue one step), so that the host has issued every step before the device
# starts the first
HEAD_START_CYCLES_PER_STEP = 1_000_000

# untimed steps queued between the spin kernel and the eager timed steps: after
# an idle gap the weight-streaming kernels slow down over the first ~7 steps of
# load (by up to ~40%) and take ~25 steps to settle
SETTLE_STEPS = 32


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


def _code_only(text):
    """C++ source without its comments and with whitespace runs collapsed, so
    that an edit of comments alone leaves the hash (and a traffic summary taken
    on that code) valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_moe_route_amd", "csrc")
    for f in ROOFLINE_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
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
        self.ev_dn = []
        self.ev_sh = []
        self.ev_layer = []

    def _timed_call(self, fn, args):
        """fn(*args) between two HIP events on the current stream (the stream
        the library launches on); returns the event pair."""
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = fn(*args)
        e1.record()
        self.moeq._check(rc, fn.__name__)
        return e0, e1

    def layer_step(self, r):
        """moe_layer_forward (moe_layer_forward_shared) on batch r with HIP
        events around the pre-marshalled C call: the whole layer as the
        library runs it (for decode batches of <= 16 assignments, the fused
        launches: routing inside gate/up, the combine inside down)."""
        import ctypes
        moeq = self.moeq
        L = moeq.lib()
        lg, x = self.batches[r % len(self.batches)]
        st = moeq._stream(x.device)
        if self.shared is None:
            args = (ctypes.byref(self.layer.c()), moeq._dptr(x), moeq._dptr(lg), self.T, self.k,
                    None, moeq._dptr(self.ids), moeq._dptr(self.w), moeq._dptr(self.out),
                    moeq._dptr(self.lws), self.lws.numel(), st)
            self.ev_layer.append(self._timed_call(L.moe_layer_forward, args))
        else:
            args = (ctypes.byref(self.layer.c()), ctypes.byref(self.shared.c()), moeq._dptr(x),
                    moeq._dptr(lg), self.T, self.k, moeq._dptr(self.ids), moeq._dptr(self.w),
                    moeq._dptr(self.out), moeq._dptr(self.lws), self.lws.numel(), st)
            self.ev_layer.append(self._timed_call(L.moe_layer_forward_shared, args))

    def step(self, r, timed):
        """One layer forward on batch r.  Untimed (warm-up and the graph
        replays that give the headline figures): the one-call layer,
        moe_layer_forward, or moe_layer_forward_shared with a shared expert
        (fused for decode batches of <= 16 assignments).
        Timed eager steps: the step-by-step calls, with HIP events around the
        gate/up and the down call (the kernel-level figures)."""
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
        st = moeq._stream(x.device)
        args = (ctypes.byref(self.layer.c()), moeq._dptr(x), moeq._dptr(perm_src),
                moeq._dptr(offsets), self.T, self.k, moeq._dptr(self.h), moeq._dptr(self.ws),
                self.ws.numel(), st)
        e0, e1 = self._timed_call(L.moe_expert_gateup_q, args)
        self.ev.append((r, e0, e1))
        args = (ctypes.byref(self.layer.c()), moeq._dptr(self.h), moeq._dptr(offsets), self.T,
                self.k, moeq._dptr(self.y), st)
        e0, e1 = self._timed_call(L.moe_expert_down_q, args)
        self.ev_dn.append((r, e0, e1))
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

    def _head_start(self, steps):
        """A spin kernel ahead of `steps` eager steps, then an event: the host
        issues every step (and its events) while the device spins, so the
        steps then run back to back as in a loop that keeps the device busy,
        and each event pair brackets its kernels rather than the host's time
        to issue them.  Returns the event after the spin."""
        spin = getattr(self.torch.cuda, "_sleep", None)
        if spin is not None:
            spin(HEAD_START_CYCLES_PER_STEP * steps)
        else:
            log("no spin kernel in this torch: the eager events include the host's issue time")
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def _end_event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def run(self, steps, warmup):
        """Eager steps: the step-by-step calls with HIP events around the
        gate/up and the down call, issued ahead of the device (a spin kernel
        first, then SETTLE_STEPS untimed steps in the same queue, so the timed
        ones run on a chip whose clocks have settled under the load).  The
        timed steps take batches warmup + SETTLE_STEPS + i.  Returns (device
        ms per step from the first timed step's start to the last one's end,
        gate/up ms per launch, down ms per launch)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i, False)
        torch.cuda.synchronize()
        self.ev, self.ev_dn, self.ev_sh = [], [], []
        self._head_start(steps + SETTLE_STEPS)
        for i in range(SETTLE_STEPS):
            self.step(warmup + i, False)
        e_start = self._end_event()
        for i in range(steps):
            self.step(warmup + SETTLE_STEPS + i, True)
        e_end = self._end_event()
        torch.cuda.synchronize()
        gu_ms = [e0.elapsed_time(e1) for _, e0, e1 in self.ev]
        dn_ms = [e0.elapsed_time(e1) for _, e0, e1 in self.ev_dn]
        return e_start.elapsed_time(e_end) / steps, gu_ms, dn_ms

    def run_layer(self, steps, warmup):
        """Eager one-call layer steps with HIP events around each call, issued
        ahead of the device (a spin kernel first, then SETTLE_STEPS untimed
        calls, as in run); the timed calls take batches warmup +
        SETTLE_STEPS + i; the ms of each timed call."""
        torch = self.torch
        for i in range(warmup):
            self.layer_step(i)
        torch.cuda.synchronize()
        self._head_start(steps + SETTLE_STEPS)
        for i in range(SETTLE_STEPS):
            self.layer_step(warmup + i)
        self.ev_layer = []
        for i in range(steps):
            self.layer_step(warmup + SETTLE_STEPS + i)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in self.ev_layer]

    def run_graph(self, steps, warmup):
        """The same steps replayed from HIP graphs, as a decode loop would run
        them: each graph holds `group` consecutive steps (each on its own input
        batch; group = the largest divisor of `steps` up to 16), so the host's
        per-graph launch cost is paid once per group.  The graphs together
        cover the batch pool a whole number of times.  The timed replays follow
        warm-up replays of at least the warm-up steps and SETTLE_STEPS steps.
        Returns (seconds, group)."""
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
        # warm-up: the W warm-up steps, and at least SETTLE_STEPS steps (after
        # the idle gap of the captures the kernels take ~25 steps of load to
        # settle; the timed replays are meant to see a decode loop's steady
        # state)
        for i in range(max((warmup + group - 1) // group, (SETTLE_STEPS + group - 1) // group)):
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
        of every touched expert, VQ codebooks once, and the shared expert's
        weights), 'routed' (the same without the shared expert) or
        'gateup'."""
        experts = self.touched[r % len(self.touched)]
        if which in ("all", "routed"):
            sh = self.shared.packed_bytes([0]) if self.shared is not None and which == "all" else 0
            return self.layer.packed_bytes(experts) + sh
        H, I = self.wl.H, self.wl.I
        tot = 0
        for e in experts:
            if self.layer.fmt_host[e] in (self.moeq.FMT_NVFP4, self.moeq.FMT_NVFP4R):
                planes = 2 if self.layer.fmt_host[e] == self.moeq.FMT_NVFP4R else 1
                tot += planes * 2 * (H * I // 2 + H * I // 16)
            elif self.moeq.vq8_rate(int(self.layer.fmt_host[e]), self.layer.vq8_m):
                m = self.moeq.vq8_rate(int(self.layer.fmt_host[e]), self.layer.vq8_m)
                tot += 2 * (H * I // 8) * m + 2 * I * 2
            else:
                tot += 2 * (H * I // 8) * 2 + 2 * I * 2
        return tot


def fused_path(layer, T, k):
    """Whether moe_layer_forward takes its fused decode path for this batch
    (a single-format layer of at most 256 experts, k <= 8 and at most 16
    assignments; a rotated one with H <= 12288): then the whole layer is two
    launches (three with a BF16 shared expert, four for a rotated layer)."""
    return (len(set(int(f) for f in layer.fmt_host)) == 1
            and (layer.rot_signs is None or layer.H <= 12288)
            and layer.E <= 256 and k <= 8 and T * k <= 16)


def measure(layer, wl, T, steps, warmup, dev, reps=16, shared=None):
    """Eager launches (HIP events around the gate/up and the down call, and
    around the one-call layer), then the same steps replayed from HIP graphs;
    the headline figures are the graph replay's, the kernel-level ones the
    eager runs'.  A shared expert runs after the routed experts on the same
    stream (its HIP events bracket its launches).

    The FFN roofline of a workload is taken over the kernels of the path its
    steps run: for a fused decode batch the one-call layer's launches (the
    routing and the combine run inside them), otherwise the gate/up and down
    kernels (+ the shared expert's); decode batches against 8 TB/s on all
    packed bytes the step reads, prefill batches against 2.5 PFLOP/s on
    6 H I flop per assignment."""
    import numpy as np
    rn = Runner(layer, wl, T, reps, dev, shared)
    ms_eager, gu_ms, dn_ms = rn.run(steps, warmup)
    lay_warm = 2
    lay_ms = rn.run_layer(steps, lay_warm)
    dt, group = rn.run_graph(steps, warmup)
    idx = list(range(steps))                          # batches of the graph replays
    idx_e = [warmup + SETTLE_STEPS + i for i in range(steps)]     # batches of the eager steps
    idx_l = [lay_warm + SETTLE_STEPS + i for i in range(steps)]   # ... of the one-call layer steps
    all_bytes = sum(rn.bytes_of(r, "all") for r in idx)
    gu_bytes = sum(rn.bytes_of(r, "gateup") for r in idx_e)
    gu_s = sum(gu_ms) / 1e3
    q = np.percentile(rn.replay_step_ms, [10, 50, 90])
    fused = fused_path(layer, T, wl.k)
    res = {
        "T": T,
        "tokens_per_s": T * steps / dt,
        "ms_per_step": dt / steps * 1e3,
        "step_ms_p10_p50_p90": [float(v) for v in q],
        "tokens_per_s_eager": T / (ms_eager / 1e3),
        "ms_per_step_eager": ms_eager,
        "steps_per_graph": group,
        "packed_GBps": all_bytes / dt / 1e9,
        "packed_frac_hbm": all_bytes / dt / 1e9 / HBM_PEAK_GBS,
        "experts_touched_mean": sum(len(rn.touched[r % reps]) for r in idx) / steps,
        "gateup_ms_mean": sum(gu_ms) / len(gu_ms),
        "down_ms_mean": sum(dn_ms) / len(dn_ms),
        "gateup_GBps": gu_bytes / gu_s / 1e9,
        "gateup_bytes_per_launch": gu_bytes / steps,
        "layer_call_ms_mean": sum(lay_ms) / len(lay_ms),
        "path": "fused" if fused else "steps",
    }
    if shared is not None:
        sh_ms = [e0.elapsed_time(e1) for _, e0, e1 in rn.ev_sh]
        sh_bytes = shared.packed_bytes([0])
        res["shared_ms_mean"] = sum(sh_ms) / len(sh_ms)
        res["shared_GBps"] = sh_bytes / (res["shared_ms_mean"] / 1e3) / 1e9
        res["shared_bytes"] = sh_bytes
    # the FFN kernels of the path the steps run
    if fused:
        ffn_ms = res["layer_call_ms_mean"]
        ffn_bytes = sum(rn.bytes_of(r, "all") for r in idx_l) / steps
    else:
        ffn_ms = res["gateup_ms_mean"] + res["down_ms_mean"] + res.get("shared_ms_mean", 0.0)
        ffn_bytes = sum(rn.bytes_of(r, "all") for r in idx_e) / steps
    res["ffn_ms"] = ffn_ms
    res["ffn_bytes_per_step"] = ffn_bytes
    res["ffn_GBps"] = ffn_bytes / (ffn_ms / 1e3) / 1e9
    if T >= PREFILL_MIN_TOKENS:
        flops = 6.0 * wl.H * wl.I * T * wl.k
        if shared is not None:
            flops += 6.0 * shared.H * shared.I * T
        res["flops_per_step"] = flops
        res["TFLOPs"] = flops / (dt / steps) / 1e12
        res["ffn_TFLOPs"] = flops / (ffn_ms / 1e3) / 1e12
        res["bound"] = "mfma"
        res["ffn_frac"] = res["ffn_TFLOPs"] / MFMA_F16_PEAK_TFLOPS
        if shared is not None:
            res["shared_TFLOPs"] = 6.0 * shared.H * shared.I * T / (res["shared_ms_mean"] / 1e3) / 1e12
    else:
        res["bound"] = "hbm"
        res["ffn_frac"] = res["ffn_GBps"] / HBM_PEAK_GBS
    return res


def compact(res):
    """The figures of one workload kept in the stdout line."""
    if "error" in res:
        return {"error": res["error"][:200]}
    return {"T": res["T"], "tok_s": round(res["tokens_per_s"], 1),
            "ms": round(res["ms_per_step"], 4), "bound": res["bound"],
            "frac": round(res["ffn_frac"], 4), "path": res["path"]}


# --------------------------------------------------------------------------

CPU_SAMPLE_TOKENS = 16
CPU_MAX_WORKERS = 16


def cpu_baseline(wl, T, ntok=CPU_SAMPLE_TOKENS):
    """The fp64 oracle on the first ntok tokens of the headline batch, its
    per-expert loop spread over a process pool on the host's cores (one BLAS
    thread per process).

    Untimed: the oracle's own encoder writes each touched expert's canonical
    NVFP4 bytes (codes and scales of gate, up and down) to a scratch folder,
    in the same pool.  Timed: routing (oracle.route_topk); then per touched
    expert, in the pool, its canonical bytes read back, decoded to fp64
    (oracle.nvfp4_dequant) and the FFN of its tokens (oracle.expert_ffn);
    then the combine (oracle.combine).  That is oracle.forward with its loop
    over experts run in parallel; the effective GB/s is the touched experts'
    packed bytes over the timed seconds."""
    import multiprocessing as mp
    import shutil
    import tempfile
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np

    import oracle
    import synth

    lg = synth.logits(wl, T, rep=0)[:ntok]
    x = synth.activations(wl, T, rep=0)[:ntok]
    ids0, _ = oracle.route_topk(lg, wl.k)
    experts = sorted(int(e) for e in np.unique(ids0))
    ncpu = len(os.sched_getaffinity(0))
    workers = max(1, min(CPU_MAX_WORKERS, ncpu, len(experts)))
    scratch = tempfile.mkdtemp(prefix="moe_oracle_")
    try:
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                 initializer=_one_blas_thread) as ex:
            list(ex.map(_oracle_encode, [(wl.name, e, scratch) for e in experts]))
            t0 = time.perf_counter()
            ids, w = oracle.route_topk(lg, wl.k)
            jobs = []
            for e in experts:
                tt, jj = np.nonzero(ids == e)
                jobs.append((e, scratch, x[tt]))
            y = np.zeros((ntok, wl.k, wl.H), dtype=np.float64)
            for (e, _, _), ye in zip(jobs, ex.map(_oracle_expert, jobs)):
                tt, jj = np.nonzero(ids == e)
                y[tt, jj] = ye
            oracle.combine(y, w)
            dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(scratch, ignore_errors=True)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nbytes = len(experts) * 3 * (wl.H * wl.I // 2 + wl.H * wl.I // 16)
    return {"value": ntok / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "GBps": nbytes / dt / 1e9,
            "sample": (f"the first {ntok} tokens of the decode T={T} batch ({len(experts)} "
                       f"experts, {nbytes / 1e9:.2f} GB packed): the fp64 oracle (route, NVFP4 "
                       f"decode from canonical bytes, FFN, combine) with its experts over "
                       f"{workers} processes of one thread on '{cpu_model}' ({ncpu} cores "
                       f"visible); {dt:.1f} s"),
            "seconds": dt}


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _oracle_encode(args):
    """The oracle's canonical NVFP4 bytes of one expert, saved to the scratch
    folder (untimed preparation of the oracle's input)."""
    import numpy as np

    import oracle
    import synth
    name, e, scratch = args
    wl = synth.WORKLOADS[name]
    for p in range(3):
        c, s = oracle.nvfp4_quantize(synth.nvfp4_source_weights(wl, e, p))
        np.save(os.path.join(scratch, f"e{e}_p{p}_codes.npy"), c)
        np.save(os.path.join(scratch, f"e{e}_p{p}_scales.npy"), s)
    return e


def _oracle_expert(args):
    """Timed: decode one expert from its canonical bytes and run the oracle
    FFN on its tokens."""
    import numpy as np

    import oracle
    e, scratch, xe = args
    W = [oracle.nvfp4_dequant(np.load(os.path.join(scratch, f"e{e}_p{p}_codes.npy")),
                              np.load(os.path.join(scratch, f"e{e}_p{p}_scales.npy")))
         for p in range(3)]
    return oracle.expert_ffn(xe, *W)


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=32, help="decode batch of the headline")
    ap.add_argument("--extra",
                    default="decode1,decode8,prefill,vq,vqprefill,vq1,vq2x8,vq3x8,vq2x8prefill,"
                            "vqmix,vqmixprefill,"
                            "mixed8,mixed32,mixedhot8,"
                            "mixedhot32,nested8,nested32,shared1,shared8,shared32,prefillshared,"
                            "rot1,rot8,rot32,"
                            "rotprefill,rotw32,rotwprefill",
                    help="comma list of other workloads to measure ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=CPU_SAMPLE_TOKENS,
                    help="tokens of the headline batch the oracle baseline runs on")
    ap.add_argument("--detail-out", default=None,
                    help="write every figure of every workload to this JSON file")
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
                # ("rotw": the wide 512-block rotation of the down input)
                wide = name.startswith("rotw")
                wr = synth.DECODE_ROT512 if wide else synth.DECODE_ROT
                nv_layer.set_rot_signs(np.stack([
                    moeq.pack_rot_signs(*[synth.rot_signs(wr, e, sd) for sd in range(5)],
                                        wr.H, wr.I) for e in range(wr.E)]), in2_block=wr.rot_in2)
                try:
                    if name.endswith("prefill"):
                        wpr = synth.Workload(wr.name.replace("decode", "prefill"), 2, 256, 8,
                                             6144, 2048, (4096,), "nvfp4", "zipf", zipf_s=1.1,
                                             rot=True, rot_in2=wr.rot_in2)
                        extra[name] = measure(nv_layer, wpr, 4096, 5, 2, dev, reps=4)
                    else:
                        T = int(name[len("rotw" if wide else "rot"):])
                        extra[name] = measure(nv_layer, wr, T, 30, 5, dev)
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
            elif name in ("vq1", "vq2x8", "vq3x8", "vq1prefill", "vq2x8prefill", "vq3x8prefill",
                          "vqmix", "vqmixprefill"):
                w8 = synth.WORKLOADS[name.replace("prefill", "")]
                log(f"building the small-codebook VQ layer {name} ...")
                lay8 = build_layer(
                    w8.E, w8.H, w8.I, synth.tier_map(w8),
                    vq8_codes=lambda e, p: (synth.vq8_codes(w8, e, p), synth.vq_scales(w8, e, p)),
                    codebooks8=[synth.vq8_codebooks(w8, p) for p in range(3)], vq8_m=w8.vq8_m,
                    device=dev, workers=16)
                if name.endswith("prefill"):
                    # the same layer at T = 4096 with the prefill routing
                    wp = synth.Workload(name, 2, w8.E, w8.k, w8.H, w8.I, (4096,), w8.fmt, "zipf",
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
        log(f"timing the oracle on a {args.cpu_tokens}-token sample ...")
        cpu = cpu_baseline(wl, args.T, args.cpu_tokens)
        cpu.pop("seconds", None)
        log("  ", json.dumps(cpu))

    achieved = head["gateup_GBps"]
    traffic = read_traffic(f"traffic_gateup_nvfp4_decode_T{args.T}.json")
    roof_ffn = {"bound": "hbm",
                "kernels": ("moe_layer_forward's fused launches" if head["path"] == "fused"
                            else "NVFP4 gate/up + down"),
                "achieved": head["ffn_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": head["ffn_frac"], "bytes_per_step": head["ffn_bytes_per_step"],
                "ms": head["ffn_ms"]}
    roof_pf = None
    pf = extra.get("prefill", {})
    if "ffn_TFLOPs" in pf:
        roof_pf = {"bound": "mfma", "kernels": "k_prefill<PfNv, 0> + k_prefill<PfNv, 1>",
                   "achieved": pf["ffn_TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "frac": pf["ffn_frac"], "ms": pf["ffn_ms"],
                   "flop_per_step": pf["flops_per_step"], "T": pf["T"]}
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
        "roofline_ffn": roof_ffn,
        "roofline_prefill": roof_pf,
        "cpu_baseline": cpu,
        "extra": {name: compact(r) for name, r in extra.items()},
    }
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump({"headline": head, "extra": extra, "line": line}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
