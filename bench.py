#!/usr/bin/env python3
"""Bench of the routed MoE decode layer on one MI355X.

A step is one pass of the whole layer over one batch of decode tokens:

    route_dispatch (router, top-k, slot lookup, grouping) -> expert_ffn_fused -> combine

The headline workload (`value`, `roofline`, `cpu_baseline`) is the largest
decode layer: 64 experts top-2, hidden 5120, expert intermediate 8192, T = 8
tokens, 4-bit g128 weights, Zipf(1.2) routing, 24 of 64 experts resident.
`per_config` repeats the measurement, each line with its own roofline and CPU
baseline, for every other decode workload: the A3B-style layer (256 experts
top-8, hidden 2048, intermediate 512, Zipf(1.1)) at T = 1, 8 and 32, and the
512-expert top-4 layer (hidden 4096, intermediate 1024, uniform routing) at
T = 1 with 4-bit and 2-bit codes.  `prefill` is the 4096-token layer on the
grouped GEMM (matrix-core utilisation).

Successive steps cycle through independently generated weight sets (like the
layers of a model), and each weight set has its own activations, so a step
finds neither its weights nor its routing in the 256 MB last-level cache from
the step before.  Inputs are resident in HBM before a timed region starts.
The layer steps are timed twice: as eager library calls, and as replays of one
HIP graph per weight set (the whole step captured once: the same kernels and
work, without the host's per-call launch cost); tokens/s is the faster of the
two, and both are in the line (eager_*, graph_*, `launch` names the one used).

Per workload:
  tokens/s      T * K / elapsed over K steps back to back (HIP events on the
                stream at the two ends only);
  roofline      the expert FFN call (one launch at the A3B-style and
                512-expert shapes; at the 64-expert shape gate/up, then the
                down call: its int8 conversion of h and the down kernel):
                algorithmic weight bytes per call (experts used * 3 * H * I *
                (bits/8 + 4/128)) over its mean duration, timed over K calls
                back to back with events at the two ends, against 8 TB/s;
                frac_of_stream is the same against a plain streaming read of
                the same byte count (moe_stream_read) timed the same way;
  cpu_baseline  the CPU oracle (single-threaded C) on the first tokens of the
                workload's first batch, pinned to one host core.
After every timed pass the FFN's and the routing's counter buffers must be
back to zero (no wait timed out); otherwise the bench exits with status 3.
With --gpus N > 1 it exits: this bench measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CONTEXT = [
    "page 'Luce Spark': ~100 tok/s at 60% expert residency vs 119 tok/s fully resident, RTX 3090, whole 33B-A3B model",
    "page 'Betelgeuse': 22 tok/s, RTX 3060 12GB, whole 68GB MoE model",
    "page 'Flash-MoE': 4.36 tok/s with a ~418 GiB/s 4-bit dequant matvec kernel, M3 Max, whole 397B model",
]

# (shape name, bits, tokens, weight sets, tokens the CPU oracle runs)
HEADLINE = ("e64", 4, 8, 2, 1)
PER_CONFIG = [("a3b", 4, 1, 4, 1), ("a3b", 4, 8, 4, 2), ("a3b", 4, 32, 4, 4),
              ("e512", 4, 1, 3, 1), ("e512", 2, 1, 3, 1)]

# FFN kernels of each decode workload (the library's choice at these sizes)
FFN_KERNELS = {
    "e64": ("ffn_gateup_xt8_kernel", "ffn_hquant_kernel", "ffn_down_rows_kernel"),
    "a3b": ("ffn_fused_dec_kernel",),
    "e512": ("ffn_fused_dec_kernel",),
}
FFN_SOURCES = {
    "e64": ("ffn_mfma.hip", "ffn_dec.hip", "mfma_ops.h", "common.h"),
    "a3b": ("ffn_dec.hip", "mfma_ops.h", "common.h"),
    "e512": ("ffn_dec.hip", "mfma_ops.h", "common.h"),
}
# the grouped GEMM's kernels and sources (its counter summary is valid for these)
GEMM_KERNELS = ("ffn_gateup_gemm_kernel", "ffn_down_gemm_kernel")
GEMM_SOURCES = ("ffn_gemm.hip", "mfma_ops.h", "common.h")
CSRC = os.path.join(ROOT, "quantized_expert_ffn_gemv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None,
                    help="run one workload 'name:bits:T' (e.g. e64:4:8) as the headline and nothing else")
    ap.add_argument("--algo", choices=["auto", "gemv", "mfma"], default="auto")
    ap.add_argument("--algo-sweep", action="store_true",
                    help="also time the decode workloads with the FFN on the vector ALUs (--algo gemv)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the A3B-style T=32 extras (warm cache, shared expert, speculative verify)")
    ap.add_argument("--no-residency", action="store_true",
                    help="skip the 64-expert layer behind the residency tiers (hot set + warm ring + host memory)")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed steps of the T=4096 prefill layer on the grouped GEMM (0 = skip)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the T=4096 prefill layer and print its measurement as one JSON line")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the runs, copy a buffer of this many MiB device to device 5 times "
                         "(the known-size kernel that scales the HBM byte counters)")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="write profiles/gemm_prefill_T4096_mfma.json from a rocprofv3 --pmc MfmaUtil folder")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "'bench.py --only W --copy-calib-mib N' into the traffic record of W under profiles/")
    return ap.parse_args()


def workload_key(name, bits, T):
    return f"{name}_q{bits}_T{T}"


def describe(shape, bits, T, sets):
    routing = "uniform routing" if shape.zipf_s is None else f"Zipf({shape.zipf_s}) routing"
    return (f"{shape.description}: T={T} tokens, hidden {shape.H}, {shape.E} experts top-{shape.k} "
            f"(renormalised gates), intermediate {shape.I}, SwiGLU, {bits}-bit g128 weights (fp16 scale+bias), "
            f"bf16 activations, {routing}, {shape.n_resident}/{shape.E} resident, {sets} rotating weight sets")


# ------------------------------------------------------------------ inputs

def upload_layer(shape, bits, seed, torch, mi, moe, with_shared=False):
    """One weight set (E routed experts; with_shared: an always-on shared expert
    of the same size as expert E of the same arrays), its router and slot table."""
    Wr, bias = mi.make_router(shape, seed)
    table = mi.make_slot_table(shape, seed)
    E = shape.E
    n = E + 1 if with_shared else E
    q, s, b = [], [], []
    for m in mi.MATRICES:
        N, K = mi.matrix_dims(shape, m)
        q.append(torch.empty((n, K // 128, N, 16 * bits), dtype=torch.uint8, device="cuda"))
        s.append(torch.empty((n, N, K // 128), dtype=torch.int16, device="cuda"))
        b.append(torch.empty((n, N, K // 128), dtype=torch.int16, device="cuda"))
    experts = mi.iter_expert_weights(shape, bits, seed)          # one expert at a time on the host
    shared = None
    if with_shared:
        one, shared_mats, gate_w = mi.make_shared_expert(shape, bits, seed)
        experts = itertools.chain(experts, [(E, shared_mats)])
    for e, mats in experts:
        for i, m in enumerate(mi.MATRICES):
            qq, ss, bb = mats[m]
            q[i][e].copy_(torch.from_numpy(moe.group_major(qq, bits)))
            s[i][e].copy_(torch.from_numpy(ss.view("int16")))
            b[i][e].copy_(torch.from_numpy(bb.view("int16")))
    dev = lambda a: torch.from_numpy(a).cuda()
    head = lambda ts, lo, hi: [t[lo:hi] for t in ts]
    if with_shared:
        shared = moe.SharedExpert(moe.QWeights(bits, head(q, E, E + 1), head(s, E, E + 1), head(b, E, E + 1)),
                                  dev(gate_w), one.I, fused_weights=moe.QWeights(bits, q, s, b))
    return dict(Wr_np=Wr, bias_np=bias, table_np=table, Wr=dev(Wr), bias=None if bias is None else dev(bias),
                table=dev(table), w=moe.QWeights(bits, head(q, 0, E), head(s, 0, E), head(b, 0, E)), shared=shared,
                seed=seed)


def timed_loop(torch, fn, steps, warmup):
    """ms of fn(0) .. fn(steps - 1) back to back after `warmup` untimed calls,
    HIP events on the current stream at the two ends only."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


class CounterFault(SystemExit):
    pass


class Runner:
    """Enqueues layer steps over rotating weight sets, one buffer set per weight
    set (so a weight set's routing outputs stay with it)."""

    def __init__(self, torch, mi, moe, shape, layers, T, algo, shared=None, acts=None):
        self.torch, self.mi, self.moe = torch, mi, moe
        self.shape, self.layers, self.T, self.algo = shape, layers, T, algo
        sh = shape
        self.d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
        self.shared = shared
        bits = layers[0]["w"].bits
        self.bufs = [moe.LayerBuffers.allocate(self.d, bits, algo, shared_rows=shared is not None)
                     for _ in layers]
        self.x, self.res, self.xb = [], [], []
        for li, L in enumerate(layers):
            xb, rb = acts(li) if acts is not None else mi.make_activations(sh.H, T, seed=1000 + L["seed"])
            self.xb.append(xb)
            self.x.append(torch.from_numpy(xb.view("int16")).cuda())
            self.res.append(torch.from_numpy(rb.view("int16")).cuda())
        self.out = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")

    def route(self, i):
        moe, n = self.moe, len(self.layers)
        L, b, x = self.layers[i % n], self.bufs[i % n], self.x[i % n]
        moe.route_dispatch(self.d, x, L["Wr"], L["bias"], True, b.logits, b.topk_ids, b.topk_w, L["table"],
                           self.shape.E, b.pair_slot, b.miss, b.n_miss, b.counts, b.offsets, b.sorted_pairs,
                           b.pair_to_row, b.active, b.n_active, b.work_list, b.n_work, sync=b.sync)

    def ffn(self, i):
        moe, n = self.moe, len(self.layers)
        L, b, x = self.layers[i % n], self.bufs[i % n], self.x[i % n]
        bits = L["w"].bits
        if self.shared is not None:
            moe.expert_ffn_fused_shared(self.d, bits, x, b.work_list, b.n_work, L["shared"].fused_weights,
                                        b.workspace, b.y_rows, b.ffn_sync, self.algo)
        else:
            moe.expert_ffn_fused(self.d, bits, x, b.work_list, b.n_work, L["w"], b.workspace, b.y_rows, b.ffn_sync,
                                 self.algo)

    def combine(self, i):
        moe, n = self.moe, len(self.layers)
        L, b, x, res = self.layers[i % n], self.bufs[i % n], self.x[i % n], self.res[i % n]
        if self.shared is None:
            moe.combine(self.d, b.y_rows, b.pair_to_row, b.topk_w, res, self.out)
        else:
            T, k = self.T, self.shape.k
            moe.combine_shared(self.d, b.y_rows, b.pair_to_row, b.topk_w, b.y_rows[T * k: T * k + T], x,
                               L["shared"].gate_w, res, self.out)

    def step(self, i):
        self.route(i)
        self.ffn(i)
        self.combine(i)

    def check_counters(self, what):
        for b in self.bufs:
            if not b.counters_clean():
                raise CounterFault(f"[bench] {what}: counters not back to zero after a timed pass "
                                   f"(FFN wait timed out: {b.ffn_timed_out()}); results of that pass are invalid")

    def experts_used(self):
        """Distinct experts per weight set for this batch (read back once, untimed)."""
        U = []
        for li in range(len(self.layers)):
            self.step(li)
            self.torch.cuda.synchronize()
            U.append(int(self.bufs[li].n_active.item()))
        return U

    def _timed(self, fn, steps, warmup):
        return timed_loop(self.torch, fn, steps, warmup)

    def timed_steps(self, steps, warmup):
        """Total ms of `steps` layer steps back to back."""
        ms = self._timed(self.step, steps, warmup)
        self.check_counters("layer steps")
        return ms

    def capture(self):
        """One HIP graph per weight set: that set's whole layer step (routing,
        FFN, combine) captured once (after eager steps); a replay redoes all of
        it on the resident inputs, without the host's per-call launch cost."""
        torch = self.torch
        self.graphs = []
        for li in range(len(self.layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(li)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def timed_graph_steps(self, steps, warmup):
        """Total ms of `steps` layer steps as graph replays (weight sets in turn)."""
        n = len(self.graphs)
        ms = self._timed(lambda i: self.graphs[i % n].replay(), steps, warmup)
        self.check_counters("graph steps")
        return ms

    def timed_ffn(self, steps, warmup):
        """Mean us of one expert FFN call: every weight set routed once into its
        own buffers, then `steps` FFN calls back to back over the weight sets in
        turn, events only before the first and after the last (no event between
        kernels adds a dispatch gap), so the figure is the kernels' own time, the
        one rocprofv3 reports."""
        for li in range(len(self.layers)):
            self.route(li)
        ms = self._timed(self.ffn, steps, warmup)
        self.check_counters("FFN calls")
        return ms / steps * 1e3


def stream_ceiling(torch, moe, nbytes, steps):
    """Mean us of one plain streaming read of nbytes (moe_stream_read), reads of
    consecutive slices of a pool at least 1 GiB and 3 x nbytes large, so no read
    finds its bytes in the last-level cache."""
    nbytes = (int(nbytes) + 4095) // 4096 * 4096
    pool_bytes = max(1 << 30, 3 * nbytes)
    n_slices = pool_bytes // nbytes
    pool = torch.empty(n_slices * nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(moe.STREAM_SINK_INTS, dtype=torch.int32, device="cuda")
    read = lambda i: moe.stream_read(pool[(i % n_slices) * nbytes:(i % n_slices + 1) * nbytes], sink)
    for i in range(3):
        read(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        read(i)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    del pool, sink
    return us


# ------------------------------------------------------- counters (traffic)

def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(key):
    return os.path.join(PROFILES, f"ffn_{key}_traffic.json")


def traffic_record(name, key):
    """HBM bytes per FFN call (all its kernels) from the committed counter
    summary of this workload, if it was taken on the current sources (else None)."""
    path = traffic_path(key)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(FFN_SOURCES[name]):
        return None
    per = rec.get("per_kernel", {})
    if not all(k in per for k in FFN_KERNELS[name]):
        return None
    return sum(per[k]["bytes_per_launch"] for k in FFN_KERNELS[name])


def _counter_rows(d):
    """Per-dispatch counter values from a rocprofv3 --pmc csv output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return out


MFMA_RECORD = "gemm_prefill_T4096_mfma.json"


def summarize_mfma(d):
    """Mean rocprofv3 `MfmaUtil` (matrix-core busy cycles summed over the SIMDs
    over the GPU's active cycles times the SIMD count, percent) per grouped-GEMM
    kernel, into profiles/gemm_prefill_T4096_mfma.json."""
    import statistics
    rows = _counter_rows(d)
    per = {}
    for k in GEMM_KERNELS:
        vals = [v for kn, c, v in rows if c == "MfmaUtil" and k in kn]
        if vals:
            per[k] = dict(mfma_util_pct=round(statistics.mean(vals), 3), dispatches=len(vals))
    rec = dict(workload="prefill layer T=4096 (bench.py --prefill-only)", per_kernel=per,
               counter="MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMD_NUM) * 100",
               sources=list(GEMM_SOURCES), source_sha256_16=source_hash(GEMM_SOURCES),
               command='rocprofv3 --kernel-include-regex "ffn_(gateup|down)_gemm" --pmc MfmaUtil -d <dir> -o run '
                       '--output-format csv -- python3 bench.py --prefill-only --prefill-steps 3')
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, MFMA_RECORD), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def mfma_record():
    """The committed MfmaUtil summary of the grouped GEMM, if taken on the current sources."""
    path = os.path.join(PROFILES, MFMA_RECORD)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(GEMM_SOURCES):
        return None
    return {k: v["mfma_util_pct"] / 100.0 for k, v in rec.get("per_kernel", {}).items()}


def summarize_counters(fetch_dir, write_dir, copy_mib, only):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per FFN kernel of the
    workload, scaled by what the same counters read for the plain copy of
    copy_mib MiB, into profiles/ffn_<workload>_traffic.json."""
    import statistics
    name, bits, T = only
    kernels = {k: k for k in FFN_KERNELS[name]} | {"copy": "copyBuffer"}
    res = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        for key, pat in kernels.items():
            vals = [v for k, c, v in rows if c == cname and pat in k]
            if key == "copy":   # the calibration copies are the largest copies of the run
                vals = sorted(vals)[-5:]
            res.setdefault(key, {})[cname] = dict(mean_kib=statistics.mean(vals) if vals else None,
                                                  dispatches=len(vals))
    copy_bytes = copy_mib * 1024 * 1024
    scale_f = copy_bytes / (res["copy"]["FETCH_SIZE"]["mean_kib"] * 1024)
    scale_w = copy_bytes / (res["copy"]["WRITE_SIZE"]["mean_kib"] * 1024)
    kern = {}
    for key in FFN_KERNELS[name]:
        if res[key]["FETCH_SIZE"]["mean_kib"] is None:
            continue
        f = res[key]["FETCH_SIZE"]["mean_kib"] * 1024 * scale_f
        w = res[key]["WRITE_SIZE"]["mean_kib"] * 1024 * scale_w
        kern[key] = dict(fetch_bytes=round(f), write_bytes=round(w), bytes_per_launch=round(f + w),
                         dispatches=res[key]["FETCH_SIZE"]["dispatches"])
    key = workload_key(name, bits, T)
    rec = dict(workload=f"{key} (bench.py --only {name}:{bits}:{T}: layer steps, then FFN calls back to back)",
               per_kernel=kern,
               copy_calibration=dict(copy_bytes=copy_bytes, fetch_scale=round(scale_f, 4),
                                     write_scale=round(scale_w, 4)),
               sources=list(FFN_SOURCES[name]), source_sha256_16=source_hash(FFN_SOURCES[name]),
               command=f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d <dir> -o run --output-format csv "
                       f"-- python3 bench.py --only {name}:{bits}:{T} --steps 20 --warmup 5 --no-cpu-baseline "
                       f"--copy-calib-mib {copy_mib}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(key), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------- CPU oracle

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(mi, shape, bits, layer0, xb, n_tok):
    """The oracle (the whole layer: router, top-k, lookup, grouping, FFN,
    combine) on the first n_tok tokens of the workload's first batch, pinned to
    one host core; tokens/s = n_tok / its time."""
    import numpy as np
    import oracle
    x = np.ascontiguousarray(xb[:n_tok])
    _, rb = mi.make_activations(shape.H, xb.shape[0], seed=1000 + layer0["seed"])
    rb = np.ascontiguousarray(rb[:n_tok])
    ids, _ = oracle.topk(oracle.router_logits(x, layer0["Wr_np"], layer0["bias_np"]), shape.k)
    U = len(np.unique(ids))
    W = mi.make_expert_weights(shape, bits, seed=layer0["seed"], experts=np.unique(ids))
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        oracle.layer(x, layer0["Wr_np"], layer0["bias_np"], W, shape.k, layer0["table_np"], shape.E, rb)
        sec = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, old)
    return dict(value=round(n_tok / sec, 3), unit="tokens/s", cores=1, kind="oracle",
                sample=f"the whole layer on the first {n_tok} token(s) of the timed batch ({n_tok * shape.k} routed "
                       f"rows, {U} experts), single-threaded C oracle (double accumulation) pinned to core {core}, "
                       f"{sec:.2f} s",
                seconds=round(sec, 3), weight_GBps=round(U * shape.bytes_per_expert(bits) / sec / 1e9, 4),
                host_cpus=os.cpu_count(), cpu_model=cpu_model())


# ------------------------------------------------------------- workloads

def measure_decode(ctx, name, bits, T, sets, n_cpu, steps, warmup, algo, with_cpu=True):
    torch, mi, moe = ctx["torch"], ctx["mi"], ctx["moe"]
    shape = mi.CONFIGS[name]
    per_expert = shape.bytes_per_expert(bits)
    layers = ctx["layers"].get((name, bits, sets))
    if layers is None:
        ctx["layers"].clear()
        torch.cuda.empty_cache()
        log(f"[bench] {name} q{bits}: uploading {sets} weight sets of {shape.E * per_expert / 1e6:.0f} MB")
        layers = [upload_layer(shape, bits, li, torch, mi, moe) for li in range(sets)]
        ctx["layers"][(name, bits, sets)] = layers
        torch.cuda.synchronize()
    r = Runner(torch, mi, moe, shape, layers, T, algo)
    U = r.experts_used()
    eager_ms = r.timed_steps(steps, warmup)
    r.capture()
    graph_ms = r.timed_graph_steps(steps, warmup)
    total_ms = min(eager_ms, graph_ms)
    launch = "one HIP graph per layer step (routing, FFN, combine), replayed" if graph_ms < eager_ms else "eager calls"
    ffn_us = r.timed_ffn(steps, warmup)
    ffn_bytes = sum(U[i % len(U)] for i in range(steps)) / steps * per_expert
    stream_us = stream_ceiling(torch, moe, ffn_bytes, steps)
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9
    stream_gbps = ffn_bytes / (stream_us * 1e-6) / 1e9
    key = workload_key(name, bits, T)
    algo_name = {moe.ALGO_AUTO: "auto", moe.ALGO_GEMV: "gemv", moe.ALGO_MFMA: "mfma"}[algo]
    out = dict(
        workload=describe(shape, bits, T, sets), key=key, H=shape.H, E=shape.E, k=shape.k, I=shape.I, T=T,
        bits=bits, group=128, weight_sets=sets, algo=algo_name,
        tokens_per_s=round(T * steps / (total_ms / 1e3), 1), ms_per_step=round(total_ms / steps, 5), launch=launch,
        eager_tokens_per_s=round(T * steps / (eager_ms / 1e3), 1), eager_ms_per_step=round(eager_ms / steps, 5),
        graph_tokens_per_s=round(T * steps / (graph_ms / 1e3), 1), graph_ms_per_step=round(graph_ms / steps, 5),
        experts_used_mean=sum(U) / len(U), experts_used_per_set=U,
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBPS, 4),
                      traffic=traffic_record(name, key) if algo == moe.ALGO_AUTO else None,
                      kernel=" + ".join(FFN_KERNELS[name]) if algo == moe.ALGO_AUTO else f"expert FFN ({algo_name})",
                      algorithmic_bytes_per_launch=round(ffn_bytes), mean_launch_us=round(ffn_us, 3),
                      launches_timed=steps,
                      stream_ceiling_GBps=round(stream_gbps, 1), frac_of_stream=round(achieved / stream_gbps, 4)),
        stream_read_us=round(stream_us, 3),
    )
    if with_cpu and ctx["cpu"]:
        log(f"[bench] {key}: timing the CPU oracle on {n_cpu} token(s)")
        out["cpu_baseline"] = cpu_baseline(mi, shape, bits, layers[0], r.xb[0], n_cpu)
    log(f"[bench] {key} ({algo_name}): {out['tokens_per_s']:.0f} tokens/s, {out['ms_per_step'] * 1e3:.1f} us/step "
        f"(eager {out['eager_ms_per_step'] * 1e3:.1f}, graph {out['graph_ms_per_step'] * 1e3:.1f}), "
        f"FFN {ffn_us:.2f} us = {achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s, "
        f"{100 * achieved / stream_gbps:.1f}% of a {stream_gbps:.0f} GB/s plain read), U={out['experts_used_mean']:.1f}")
    del r
    return out


def measure_residency(ctx, steps, warmup, n_hot=24, n_warm=8, T=8, batches=64):
    """The 64-expert T=8 layer with its experts behind the residency tiers:
    every expert in pinned host memory, the hot set (24 of 64) calibrated on
    the GPU from the routing counts of 1024 calibration tokens, a warm ring of
    n_warm slots (copies from host memory on a second stream while the FFN of
    the resident experts runs).  Steps cycle through `batches` distinct token
    batches, so the ring keeps missing at the rate the routing gives.  Beside
    it: the same batches with every expert in HBM."""
    torch, mi, moe = ctx["torch"], ctx["mi"], ctx["moe"]
    shape, bits = mi.CONFIGS["e64"], 4
    ctx["layers"].clear()
    torch.cuda.empty_cache()
    E = shape.E
    log(f"[bench] residency: {E} experts of {shape.bytes_per_expert(bits) / 1e6:.1f} MB into pinned host memory")
    hq, hs, hb = [], [], []
    for m in mi.MATRICES:
        N, K = mi.matrix_dims(shape, m)
        hq.append(torch.empty((E, K // 128, N, 16 * bits), dtype=torch.uint8, pin_memory=True))
        hs.append(torch.empty((E, N, K // 128), dtype=torch.int16, pin_memory=True))
        hb.append(torch.empty((E, N, K // 128), dtype=torch.int16, pin_memory=True))
    for e, mats in mi.iter_expert_weights(shape, bits, 0):
        for i, m in enumerate(mi.MATRICES):
            qq, ss, bb = mats[m]
            hq[i][e].copy_(torch.from_numpy(moe.group_major(qq, bits)))
            hs[i][e].copy_(torch.from_numpy(ss.view("int16")))
            hb[i][e].copy_(torch.from_numpy(bb.view("int16")))
    host = moe.QWeights(bits, hq, hs, hb)
    full = moe.QWeights(bits, [t.cuda() for t in hq], [t.cuda() for t in hs], [t.cuda() for t in hb])
    Wr, bias = mi.make_router(shape, 0)
    Wr_d, bias_d = torch.from_numpy(Wr).cuda(), None if bias is None else torch.from_numpy(bias).cuda()
    # calibration: 1024 tokens (seed 1) routed in batches of 64, counted on the device
    dc = moe.dims(64, shape.H, shape.I, E, shape.k)
    cbuf = moe.LayerBuffers.allocate(dc, bits)
    xc, _ = mi.make_activations(shape.H, 1024, 1)
    none = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    freq = torch.zeros(E, dtype=torch.int32, device="cuda")
    for b in range(0, 1024, 64):
        moe.route_dispatch(dc, torch.from_numpy(xc[b:b + 64].view("int16")).cuda(), Wr_d, bias_d, True, cbuf.logits,
                           cbuf.topk_ids, cbuf.topk_w, none, E, cbuf.pair_slot, cbuf.miss, cbuf.n_miss, cbuf.counts,
                           cbuf.offsets, cbuf.sorted_pairs, cbuf.pair_to_row, cbuf.active, cbuf.n_active,
                           cbuf.work_list, cbuf.n_work, sync=cbuf.sync)
        moe.route_counts(dc, cbuf.counts, freq)
    hot = torch.empty(n_hot, dtype=torch.int32, device="cuda")
    moe.hot_set(dc, freq, n_hot, hot)
    d = moe.dims(T, shape.H, shape.I, E, shape.k)
    res = moe.ResidentExperts.allocate(d, bits, host, n_hot=n_hot, n_slots=n_hot + n_warm)
    res.install(hot)
    buf = moe.LayerBuffers.allocate(d, bits)
    ref = moe.LayerBuffers.allocate(d, bits)
    xs, rs = [], []
    for i in range(batches):
        xb, rb = mi.make_activations(shape.H, T, seed=3000 + i)
        xs.append(torch.from_numpy(xb.view("int16")).cuda())
        rs.append(torch.from_numpy(rb.view("int16")).cuda())
    out = torch.empty((T, shape.H), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    all_res = torch.arange(E, dtype=torch.int32, device="cuda")
    state = {"step": 0}

    def tiered(i):
        state["step"] += 1
        moe.resident_layer_forward(buf, res, xs[i % batches], Wr_d, bias_d, rs[i % batches], out, state["step"],
                                   copy_stream=side)

    def resident(i):
        moe.layer_forward(ref, xs[i % batches], Wr_d, bias_d, full, all_res, E, rs[i % batches], out)

    # misses and copies per step, counted in an untimed pass over every batch
    copies = cold = misses = 0
    for i in range(batches):
        tiered(i)
        torch.cuda.synchronize()
        misses += int(buf.n_miss.item())
        copies += int(res.n_copy.item())
        cold += int(res.list_counts[2].item())
    t_ms = timed_loop(torch, tiered, steps, warmup)
    if not buf.counters_clean():
        raise CounterFault("[bench] residency steps: counters not back to zero")
    a_ms = timed_loop(torch, resident, steps, warmup)
    per = shape.bytes_per_expert(bits)
    out_d = dict(workload=f"64-expert layer T={T} behind residency tiers: {n_hot} hot experts (calibrated on the GPU "
                          f"from 1024 tokens), a {n_warm}-slot warm ring, all {E} experts in pinned host memory, "
                          f"{batches} distinct batches",
                 n_hot=n_hot, n_warm=n_warm, tokens_per_s=round(T * steps / (t_ms / 1e3), 1),
                 ms_per_step=round(t_ms / steps, 4), misses_per_step=round(misses / batches, 3),
                 copies_per_step=round(copies / batches, 3), cold_entries_per_step=round(cold / batches, 3),
                 copy_MB_per_step=round(copies / batches * per / 1e6, 1),
                 all_resident_tokens_per_s=round(T * steps / (a_ms / 1e3), 1),
                 all_resident_ms_per_step=round(a_ms / steps, 4))
    log(f"[bench] residency: {out_d['tokens_per_s']:.0f} tokens/s ({out_d['ms_per_step']:.3f} ms/step), "
        f"{out_d['misses_per_step']} misses and {out_d['copies_per_step']} copies per step; "
        f"all resident {out_d['all_resident_tokens_per_s']:.0f} tokens/s")
    del res, buf, ref, full, host, hq, hs, hb
    torch.cuda.empty_cache()
    return out_d


def measure_stack(torch, mi, moe, shape, layers, T, steps, warmup):
    """A decode step through the weight sets as a stack of layers (layer l's
    output is layer l+1's input and residual), enqueued call by call and as one
    HIP graph per token step (moe.stack_forward captured once, replayed)."""
    d = moe.dims(T, shape.H, shape.I, shape.E, shape.k)
    bits = layers[0]["w"].bits
    bufs = [moe.LayerBuffers.allocate(d, bits) for _ in layers]
    outs = [torch.empty((T, shape.H), dtype=torch.int16, device="cuda") for _ in layers]
    x = torch.from_numpy(mi.make_activations(shape.H, T, seed=3000)[0].view("int16")).cuda()
    sl = [moe.StackLayer(L["Wr"], L["bias"], L["w"], L["table"], shape.E) for L in layers]
    run = lambda i: moe.stack_forward(bufs, x, sl, outs)
    eager_ms = timed_loop(torch, run, steps, warmup)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(0)
    torch.cuda.synchronize()
    graph_ms = timed_loop(torch, lambda i: graph.replay(), steps, warmup)
    for b in bufs:
        if not b.counters_clean():
            raise CounterFault("[bench] stack: counters not back to zero after the timed replays")
    n = len(layers)
    res = dict(layers=n, T=T, eager_us_per_token_step=round(eager_ms / steps * 1e3, 2),
               graph_us_per_token_step=round(graph_ms / steps * 1e3, 2),
               graph_us_per_layer=round(graph_ms / steps * 1e3 / n, 2),
               graph_tokens_per_s=round(T / (graph_ms / steps / 1e3), 1))
    del graph, bufs, outs
    return res


def measure_a3b_extras(ctx, steps, warmup):
    """The A3B-style T=32 step with an always-on shared expert (inside the routed
    FFN launch, sigmoid gate fused into the combine), on a speculative-verify
    batch (8 sequences x 4 correlated drafts), and warm (one weight set)."""
    torch, mi, moe = ctx["torch"], ctx["mi"], ctx["moe"]
    shape, T, bits = mi.CONFIGS["a3b"], 32, 4
    ctx["layers"].clear()
    torch.cuda.empty_cache()
    layers = [upload_layer(shape, bits, li, torch, mi, moe, with_shared=True) for li in range(4)]
    out = {}
    base = Runner(torch, mi, moe, shape, layers, T, moe.ALGO_AUTO)
    base.experts_used()
    base_ms = base.timed_steps(steps, warmup) / steps
    sh = Runner(torch, mi, moe, shape, layers, T, moe.ALGO_AUTO, shared=True)
    sh.experts_used()
    sh_ms = sh.timed_steps(steps, warmup) / steps
    out["shared_expert"] = dict(I_shared=shape.I, tokens_per_s=round(T / (sh_ms / 1e3), 1),
                                ms_per_step=round(sh_ms, 5), added_us_per_step=round((sh_ms - base_ms) * 1e3, 2))
    n_seq = T // 4
    sv = Runner(torch, mi, moe, shape, layers, T, moe.ALGO_AUTO,
                acts=lambda li: mi.make_spec_verify_activations(shape.H, n_seq, 4, seed=2000 + li))
    U_sv = sv.experts_used()
    sv_ms = sv.timed_steps(steps, warmup) / steps
    out["spec_verify"] = dict(sequences=n_seq, drafts_per_sequence=4, rho=0.8, tokens_per_s=round(T / (sv_ms / 1e3), 1),
                              ms_per_step=round(sv_ms, 5), experts_used_mean=sum(U_sv) / len(U_sv))
    warm = Runner(torch, mi, moe, shape, layers[:1], T, moe.ALGO_AUTO)
    warm.experts_used()
    w_ms = warm.timed_steps(steps, warmup) / steps
    out["warm_one_weight_set"] = dict(tokens_per_s=round(T / (w_ms / 1e3), 1), ms_per_step=round(w_ms, 5))
    out["cold_ms_per_step"] = round(base_ms, 5)
    log(f"[bench] a3b T=32 extras: shared expert +{out['shared_expert']['added_us_per_step']} us/step; "
        f"spec verify {out['spec_verify']['tokens_per_s']:.0f} tokens/s; warm {out['warm_one_weight_set']['tokens_per_s']:.0f}")
    out["stack"] = [measure_stack(torch, mi, moe, shape, layers, t, steps, warmup) for t in (1, 8)]
    for s in out["stack"]:
        log(f"[bench] a3b stack of {s['layers']} layers, T={s['T']}: {s['graph_us_per_token_step']} us per token step "
            f"as one graph ({s['graph_us_per_layer']} us/layer), {s['eager_us_per_token_step']} us call by call")
    del base, sh, sv, warm, layers
    ctx["layers"].clear()
    torch.cuda.empty_cache()
    return out


def measure_prefill(ctx, steps, warmup):
    """The prefill-shape layer (T = 4096) with the FFN on the grouped GEMM:
    matrix-core utilisation = useful FFN flops / FFN kernel time / bf16 peak."""
    torch, mi, moe = ctx["torch"], ctx["mi"], ctx["moe"]
    shape = mi.CONFIGS["prefill"]
    T = shape.tokens[0]
    ctx["layers"].clear()
    torch.cuda.empty_cache()
    log(f"[bench] prefill: uploading {shape.E * shape.bytes_per_expert(4) / 1e6:.0f} MB, T={T}")
    layer = upload_layer(shape, 4, 0, torch, mi, moe)
    r = Runner(torch, mi, moe, shape, [layer], T, moe.ALGO_AUTO)
    U = r.experts_used()[0]
    total_ms = r.timed_steps(steps, warmup)
    d, b, L = r.d, r.bufs[0], layer
    r.route(0)
    gate_ms = r._timed(lambda i: moe.expert_gateup(d, 4, r.x[0], b.work_list, b.n_work, L["w"], b.workspace,
                                                   moe.ALGO_AUTO), steps, 2)
    down_ms = r._timed(lambda i: moe.expert_down(d, 4, b.work_list, b.n_work, L["w"], b.workspace, b.y_rows,
                                                 moe.ALGO_AUTO), steps, 2)
    P = T * shape.k
    gate_flop, down_flop = 2.0 * P * 2 * shape.H * shape.I, 2.0 * P * shape.H * shape.I
    g_s, d_s = gate_ms / 1e3 / steps, down_ms / 1e3 / steps
    util = (gate_flop + down_flop) / (g_s + d_s) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    del r, layer
    torch.cuda.empty_cache()
    out = dict(workload=f"prefill layer T={T}: hidden {shape.H}, {shape.E} experts top-{shape.k}, "
                        f"intermediate {shape.I}, 4-bit g128, Zipf(1.0) routing",
               algo="grouped GEMM (AUTO)", steps=steps, experts_used=U,
               tokens_per_s=round(T / (total_ms / 1e3 / steps), 1), ms_per_step=round(total_ms / steps, 4),
               gateup_us=round(g_s * 1e6, 2), down_us=round(d_s * 1e6, 2),
               ffn_tflops=round((gate_flop + down_flop) / (g_s + d_s) / 1e12, 1),
               gateup_tflops=round(gate_flop / g_s / 1e12, 1), down_tflops=round(down_flop / d_s / 1e12, 1),
               mfma_util=round(util, 4), mfma_peak_tflops=MFMA_BF16_PEAK_TFLOPS,
               mfma_busy_counter=mfma_record(),
               note="mfma_util: useful FFN flops (2*T*k*3*H*I) over the two GEMM kernels' time, each timed over "
                    "the steps back to back, against the dense bf16 peak; mfma_busy_counter: the fraction of "
                    "cycles the matrix cores were busy per kernel (rocprofv3 MfmaUtil, "
                    "profiles/gemm_prefill_T4096_mfma.json; null when taken on other sources)")
    log(f"[bench] prefill: {out['tokens_per_s']:.0f} tokens/s, FFN {out['ffn_tflops']} TFLOP/s "
        f"({100 * util:.1f}% of bf16 MFMA peak)")
    return out


def main():
    args = parse()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_counters:
        if not args.only:
            raise SystemExit("--summarize-counters needs --only name:bits:T (the workload the counters ran)")
        name, bits, T = args.only.split(":")
        summarize_counters(*args.summarize_counters, args.copy_calib_mib or 256, (name, int(bits), int(T)))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU expert-parallel design is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi
    import quantized_expert_ffn_gemv_amd as moe

    torch.cuda.set_device(0)
    moe.lib()
    algo = {"auto": moe.ALGO_AUTO, "gemv": moe.ALGO_GEMV, "mfma": moe.ALGO_MFMA}[args.algo]
    ctx = dict(torch=torch, mi=mi, moe=moe, layers={}, cpu=not args.no_cpu_baseline)
    if args.prefill_only:
        print(json.dumps({"prefill": measure_prefill(ctx, max(args.prefill_steps, 1), 3)}), flush=True)
        return

    if args.only:
        name, bits, T = args.only.split(":")
        head_spec = next((c for c in [HEADLINE] + PER_CONFIG if c[:3] == (name, int(bits), int(T))),
                         (name, int(bits), int(T), 2, 1))
        per_specs = []
    else:
        head_spec, per_specs = HEADLINE, PER_CONFIG
    try:
        head = measure_decode(ctx, *head_spec, args.steps, args.warmup, algo)
        per = [measure_decode(ctx, *spec, args.steps, args.warmup, algo) for spec in per_specs]
        algo_sweep = []
        if args.algo_sweep:
            for spec in [head_spec] + per_specs:
                algo_sweep.append(measure_decode(ctx, *spec, args.steps, args.warmup, moe.ALGO_GEMV, with_cpu=False))
        extras = None if (args.only or args.no_extras) else measure_a3b_extras(ctx, max(args.steps // 2, 10),
                                                                               max(args.warmup // 2, 2))
        residency = None
        if not (args.only or args.no_residency):
            residency = measure_residency(ctx, max(args.steps // 4, 10), max(args.warmup // 2, 2))
        prefill = None
        if args.prefill_steps > 0 and not args.only:
            prefill = measure_prefill(ctx, args.prefill_steps, 3)
    except CounterFault as e:
        print(str(e), file=sys.stderr, flush=True)
        sys.exit(3)

    if args.copy_calib_mib:
        n = args.copy_calib_mib * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    config = {k: head[k] for k in ("workload", "H", "E", "k", "I", "T", "bits", "group", "weight_sets", "algo")}
    config.update(ffn="one call (expert_ffn_fused)", launch=head["launch"], parallelism="none (one GPU)")
    result = {
        "metric": "MoE-layer decode tokens/s + weight-stream HBM GB/s (% of MI355X peak)",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "experts_used_mean": head["experts_used_mean"],
        "stream_read_us": head["stream_read_us"],
        "per_config": per,
        "algo_gemv": algo_sweep or None,
        "a3b_T32_extras": extras,
        "residency": residency,
        "prefill": prefill,
        "context_not_comparable": CONTEXT,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
