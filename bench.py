#!/usr/bin/env python3
"""Bench of the routed MoE decode layer on one MI355X.

Workload: the A3B-style decode layer (hidden 2048, 256 experts, top-8 with
renormalised gates, expert intermediate 512, SwiGLU, 4-bit weights with fp16
scale and bias per group of 128, Zipf(1.1) expert popularity), a batch of
--tokens decode tokens (default 32).  A step is one pass of the whole layer:

    route_dispatch (router, top-k, slot lookup, grouping) -> expert_ffn_fused -> combine

(--ffn split: expert_gateup -> expert_down in place of expert_ffn_fused).

Successive steps cycle through --layers independently generated weight sets
(like successive layers of a model; 4 x 428 MB by default), so the weights
cannot stay in the 256 MB last-level cache and every step streams them from
HBM.  Inputs are resident in HBM before the timed region starts.  The timed
steps are eager library calls (--launch graph replays one captured HIP graph
per weight set instead; every kernel of the step runs at each replay).

Printed: one JSON line with
  value         tokens/s over the K timed steps (tokens * K / elapsed);
  roofline      the FFN kernel (the one-launch gate/up + down kernel; with
                --ffn split or --algo gemv, the gate/up kernel): algorithmic
                weight bytes per launch (experts used * 3 * I * H * (bits/8 +
                4/128), or 2 * ... for gate/up alone) over its mean duration,
                timed with HIP events around each launch on the stream it runs
                on, against the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle (single-threaded C) timed on one full step of
                weight set 0 on this host.
With --gpus N > 1 it exits: this bench measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CONTEXT = [
    "page 'Luce Spark': ~100 tok/s at 60% expert residency vs 119 tok/s fully resident, RTX 3090, whole 33B-A3B model",
    "page 'Betelgeuse': 22 tok/s, RTX 3060 12GB, whole 68GB MoE model",
    "page 'Flash-MoE': 4.36 tok/s with a ~418 GiB/s 4-bit dequant matvec kernel, M3 Max, whole 397B model",
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=32)
    ap.add_argument("--layers", type=int, default=4, help="rotating weight sets")
    ap.add_argument("--sweep", default="1,8", help="extra token counts timed after the main run ('none' = none)")
    ap.add_argument("--algo", choices=["auto", "gemv", "mfma"], default="auto")
    ap.add_argument("--ffn", choices=["fused", "split"], default="fused",
                    help="expert FFN as one call (expert_ffn_fused) or as expert_gateup + expert_down")
    ap.add_argument("--launch", choices=["eager", "graph"], default="eager",
                    help="timed steps as eager library calls, or as replays of one captured HIP graph per weight "
                         "set (each replays every kernel of the step; measured slower here)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shared-expert", action="store_true",
                    help="skip the extra measurement of the step with a shared expert")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed steps of the T=4096 prefill layer on the grouped GEMM (0 = skip)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the runs, copy a buffer of this many MiB device to device 5 times "
                         "(the known-size kernel that scales the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "'bench.py --copy-calib-mib N' into the traffic record under profiles/")
    return ap.parse_args()


def upload_layer(shape, bits, seed, torch, mi, moe):
    """One weight set: the E routed experts, then an always-on shared expert of
    the same size as expert E of the same arrays (`w` views the routed ones;
    `shared` holds the shared expert both ways and its gate row)."""
    Wr, bias = mi.make_router(shape, seed)
    table = mi.make_slot_table(shape, seed)
    E = shape.E
    q, s, b = [], [], []
    for m in mi.MATRICES:
        N, K = mi.matrix_dims(shape, m)
        q.append(torch.empty((E + 1, K // 128, N, 16 * bits), dtype=torch.uint8, device="cuda"))
        s.append(torch.empty((E + 1, N, K // 128), dtype=torch.int16, device="cuda"))
        b.append(torch.empty((E + 1, N, K // 128), dtype=torch.int16, device="cuda"))
    one, shared_mats, gate_w = mi.make_shared_expert(shape, bits, seed)
    for e, mats in list(mi.iter_expert_weights(shape, bits, seed)) + [(E, shared_mats)]:
        for i, m in enumerate(mi.MATRICES):
            qq, ss, bb = mats[m]
            q[i][e].copy_(torch.from_numpy(moe.group_major(qq, bits)))
            s[i][e].copy_(torch.from_numpy(ss.view("int16")))
            b[i][e].copy_(torch.from_numpy(bb.view("int16")))
    dev = lambda a: torch.from_numpy(a).cuda()
    head = lambda ts, lo, hi: [t[lo:hi] for t in ts]
    shared = moe.SharedExpert(moe.QWeights(bits, head(q, E, E + 1), head(s, E, E + 1), head(b, E, E + 1)),
                              dev(gate_w), one.I, fused_weights=moe.QWeights(bits, q, s, b))
    return dict(Wr_np=Wr, bias_np=bias, table_np=table, Wr=dev(Wr), bias=None if bias is None else dev(bias),
                table=dev(table), w=moe.QWeights(bits, head(q, 0, E), head(s, 0, E), head(b, 0, E)), shared=shared)


class Runner:
    """Enqueues layer steps over rotating weight sets; optional events around the
    FFN halves; optionally a shared expert per weight set (its FFN first, its
    gate in the combine)."""

    def __init__(self, torch, mi, moe, shape, layers, T, algo, fused_ffn=False, shared=None, one_launch=True,
                 acts=None):
        self.torch, self.mi, self.moe = torch, mi, moe
        self.shape, self.layers, self.T, self.algo = shape, layers, T, algo
        self.fused_ffn = fused_ffn
        sh = shape
        self.d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
        self.shared = shared
        self.one_launch = shared is not None and one_launch and fused_ffn
        self.buf = moe.LayerBuffers.allocate(self.d, layers[0]["w"].bits, algo, shared_rows=self.one_launch)
        if shared is not None:
            self.sbuf = moe.SharedBuffers.allocate(T, sh.H, shared[0].I, layers[0]["w"].bits, algo)
        self.x, self.res = [], []
        for li in range(len(layers)):
            xb, rb = acts(li) if acts is not None else mi.make_activations(sh.H, T, seed=1000 + li)
            self.x.append(torch.from_numpy(xb.view("int16")).cuda())
            self.res.append(torch.from_numpy(rb.view("int16")).cuda())
        self.out = torch.empty((T, sh.H), dtype=torch.int16, device="cuda")

    def step(self, i, ev=None):
        moe, b, d = self.moe, self.buf, self.d
        L = self.layers[i % len(self.layers)]
        x, res = self.x[i % len(self.layers)], self.res[i % len(self.layers)]
        bits = L["w"].bits
        if self.shared is not None:
            S, sb = self.shared[i % len(self.shared)], self.sbuf
            if not self.one_launch:
                moe.expert_ffn_fused(sb.d, bits, x, sb.buf.work_list, sb.buf.n_work, S.weights, sb.buf.workspace,
                                     sb.buf.y_rows, sb.buf.ffn_sync, self.algo)
        moe.route_dispatch(d, x, L["Wr"], L["bias"], True, b.logits, b.topk_ids, b.topk_w, L["table"],
                           self.shape.E, b.pair_slot, b.miss, b.n_miss, b.counts, b.offsets, b.sorted_pairs,
                           b.pair_to_row, b.active, b.n_active, b.work_list, b.n_work, sync=b.sync)
        if ev is not None:
            ev[0].record()
        if self.one_launch:
            moe.expert_ffn_fused_shared(d, bits, x, b.work_list, b.n_work, S.fused_weights, b.workspace, b.y_rows,
                                        b.ffn_sync, self.algo)
            if ev is not None:
                ev[1].record()
        elif self.fused_ffn:
            moe.expert_ffn_fused(d, bits, x, b.work_list, b.n_work, L["w"], b.workspace, b.y_rows, b.ffn_sync,
                                 self.algo)
            if ev is not None:
                ev[1].record()
        else:
            moe.expert_gateup(d, bits, x, b.work_list, b.n_work, L["w"], b.workspace, self.algo)
            if ev is not None:
                ev[1].record()
            moe.expert_down(d, bits, b.work_list, b.n_work, L["w"], b.workspace, b.y_rows, self.algo)
        if ev is not None:
            ev[2].record()
        if self.shared is None:
            moe.combine(d, b.y_rows, b.pair_to_row, b.topk_w, res, self.out)
        else:
            T, k = self.T, self.shape.k
            ys = b.y_rows[T * k: T * k + T] if self.one_launch else sb.buf.y_rows
            moe.combine_shared(d, b.y_rows, b.pair_to_row, b.topk_w, ys, x, S.gate_w, res, self.out, sb.gate_out)

    def timed_ffn_launches(self, steps, warmup):
        """Mean duration (us) of the one-launch FFN alone: every weight set is
        routed once into a buffer set of its own, then `steps` FFN launches run
        back to back over the weight sets in turn, with HIP events on their
        stream only before the first and after the last (no event between
        kernels adds a dispatch gap), so the figure is the kernel's own
        average, the one rocprofv3 reports."""
        torch, moe, d = self.torch, self.moe, self.d
        n = len(self.layers)
        bits = self.layers[0]["w"].bits
        bufs = [moe.LayerBuffers.allocate(d, bits, self.algo) for _ in range(n)]
        for li in range(n):
            L, b = self.layers[li], bufs[li]
            moe.route_dispatch(d, self.x[li], L["Wr"], L["bias"], True, b.logits, b.topk_ids, b.topk_w, L["table"],
                               self.shape.E, b.pair_slot, b.miss, b.n_miss, b.counts, b.offsets, b.sorted_pairs,
                               b.pair_to_row, b.active, b.n_active, b.work_list, b.n_work, sync=b.sync)

        def launch(i):
            L, b = self.layers[i % n], bufs[i % n]
            moe.expert_ffn_fused(d, bits, self.x[i % n], b.work_list, b.n_work, L["w"], b.workspace, b.y_rows,
                                 b.ffn_sync, self.algo)
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            launch(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps * 1e3

    def experts_used(self):
        """Distinct experts per weight set for this batch (read back once, untimed)."""
        U = []
        for li in range(len(self.layers)):
            self.step(li)
            self.torch.cuda.synchronize()
            U.append(int(self.buf.n_active.item()))
        return U

    def capture(self):
        """One HIP graph per weight set, each holding a whole layer step (its
        kernels replay on the same buffers; nothing is allocated or copied)."""
        torch = self.torch
        self.graphs = []
        for li in range(len(self.layers)):
            self.step(li)                                     # eager first: caches launch sizes
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(li)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def timed_graphs(self, steps, warmup):
        """(total ms, wall s) of `steps` graph replays, weight sets in turn."""
        torch = self.torch
        for i in range(warmup):
            self.graphs[i % len(self.graphs)].replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t0.record()
        for i in range(steps):
            self.graphs[i % len(self.graphs)].replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), time.perf_counter() - wall0

    def timed(self, steps, warmup, with_events=True):
        """(total ms, wall s, per-step ms from event 0 to 1, from 1 to 2): with
        the FFN as one call, 0 -> 1 is that call and 1 -> 2 is empty."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)] if with_events else None
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for i in range(steps):
            self.step(i, evs[i] if evs else None)
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t0.elapsed_time(t1)
        gate_ms = [e[0].elapsed_time(e[1]) for e in evs] if evs else None
        down_ms = [e[1].elapsed_time(e[2]) for e in evs] if evs else None
        return total_ms, wall, gate_ms, down_ms


CSRC = os.path.join(ROOT, "quantized_expert_ffn_gemv_amd", "csrc")

# The FFN kernels the default decode workload runs, per --algo (auto and mfma
# take the LDS-staged decode kernels at these sizes), and the sources they are
# built from.
FFN_KERNELS = {
    "mfma": dict(gateup="ffn_gateup_dec_kernel", down="ffn_down_dec_kernel", fused="ffn_fused_dec_kernel",
                 sources=("ffn_dec.hip", "mfma_ops.h", "common.h")),
    "gemv": dict(gateup="ffn_gateup_gemv_kernel", down="ffn_down_gemv_kernel",
                 sources=("ffn_gemv.hip", "common.h")),
}
FFN_KERNELS["auto"] = FFN_KERNELS["mfma"]


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "ffn_a3b_T32_traffic.json")


def traffic_record(algo, key):
    """HBM bytes per launch of FFN kernel `key` (gateup, down, fused) from the
    committed counter summary, if it was taken on the current sources (else None)."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        rec = json.load(f)
    k = FFN_KERNELS[algo]
    if key not in k or rec.get("source_sha256_16") != source_hash(k["sources"]):
        return None
    return rec.get("per_kernel", {}).get(k[key], {}).get("bytes_per_launch")


MFMA_BF16_PEAK_TFLOPS = 2500.0


def measure_prefill(torch, mi, moe, steps, warmup):
    """The prefill-shape layer (T = 4096) with the FFN on the grouped GEMM:
    matrix-core utilisation = useful FFN flops / FFN kernel time / bf16 peak."""
    shape = mi.CONFIGS["prefill"]
    T = shape.tokens[0]
    log(f"[bench] prefill: uploading {shape.E * shape.bytes_per_expert(4) / 1e6:.0f} MB, T={T}")
    layer = upload_layer(shape, 4, seed=0, torch=torch, mi=mi, moe=moe)
    r = Runner(torch, mi, moe, shape, [layer], T, moe.ALGO_AUTO)
    U = r.experts_used()[0]
    total_ms, _, gate_ms, down_ms = r.timed(steps, warmup)
    P = T * shape.k
    gate_flop, down_flop = 2.0 * P * 2 * shape.H * shape.I, 2.0 * P * shape.H * shape.I
    g_s, d_s = sum(gate_ms) / 1e3 / steps, sum(down_ms) / 1e3 / steps
    util = (gate_flop + down_flop) / (g_s + d_s) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    del r, layer
    torch.cuda.empty_cache()
    return dict(workload=f"prefill layer T={T}: hidden {shape.H}, {shape.E} experts top-{shape.k}, "
                         f"intermediate {shape.I}, 4-bit g128, Zipf(1.0) routing",
                algo="grouped GEMM (AUTO)", steps=steps, experts_used=U,
                tokens_per_s=round(T / (total_ms / 1e3 / steps), 1), ms_per_step=round(total_ms / steps, 4),
                gateup_us=round(g_s * 1e6, 2), down_us=round(d_s * 1e6, 2),
                ffn_tflops=round((gate_flop + down_flop) / (g_s + d_s) / 1e12, 1),
                gateup_tflops=round(gate_flop / g_s / 1e12, 1), down_tflops=round(down_flop / d_s / 1e12, 1),
                mfma_util=round(util, 4), mfma_peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                note="useful FFN flops (2*T*k*3*H*I) only; the exact-operand scheme also runs all-ones "
                     "MFMAs for the group sums and two h planes in the down GEMM")


def traffic_kernels(algo):
    k = FFN_KERNELS[algo]
    return {key: k[key] for key in ("gateup", "down", "fused") if key in k} | {"copy": "copyBuffer"}


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


def summarize_counters(fetch_dir, write_dir, copy_mib, algo="auto"):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by
    what the same counters read for the plain copy of copy_mib MiB."""
    import statistics
    res = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        for key, pat in traffic_kernels(algo).items():
            vals = [v for k, c, v in rows if c == cname and pat in k]
            if key == "copy":   # the calibration copies are the largest copies of the run
                vals = sorted(vals)[-5:]
            res.setdefault(key, {})[cname] = dict(mean_kib=statistics.mean(vals) if vals else None,
                                                  dispatches=len(vals))
    copy_bytes = copy_mib * 1024 * 1024
    f_copy = res["copy"]["FETCH_SIZE"]["mean_kib"] * 1024
    w_copy = res["copy"]["WRITE_SIZE"]["mean_kib"] * 1024
    scale_f, scale_w = copy_bytes / f_copy, copy_bytes / w_copy
    kern = {}
    k = FFN_KERNELS[algo]
    for key in traffic_kernels(algo):
        if key == "copy" or res[key]["FETCH_SIZE"]["mean_kib"] is None:
            continue
        f = res[key]["FETCH_SIZE"]["mean_kib"] * 1024 * scale_f
        w = res[key]["WRITE_SIZE"]["mean_kib"] * 1024 * scale_w
        kern[k[key]] = dict(fetch_bytes=round(f), write_bytes=round(w), bytes_per_launch=round(f + w),
                            dispatches=res[key]["FETCH_SIZE"]["dispatches"])
    rec = dict(workload="a3b T=32 (bench.py default: the one-launch FFN timed, then the two-launch FFN)",
               per_kernel=kern,
               copy_calibration=dict(copy_bytes=copy_bytes, fetch_scale=round(scale_f, 4),
                                     write_scale=round(scale_w, 4)),
               sources=list(k["sources"]), source_sha256_16=source_hash(k["sources"]),
               command="rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d <dir> -o run --output-format csv "
                       "-- python3 bench.py --steps 20 --warmup 5 --sweep=none --no-cpu-baseline --prefill-steps 0 "
                       f"--no-shared-expert --copy-calib-mib {copy_mib}")
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(mi, shape, layer0, T):
    """Oracle timed on one full layer step of weight set 0 (same inputs as the GPU),
    pinned to one host core for the timed call."""
    import numpy as np
    import oracle
    xb, rb = mi.make_activations(shape.H, T, seed=1000)
    logits = oracle.router_logits(xb, layer0["Wr_np"], layer0["bias_np"])
    ids, _ = oracle.topk(logits, shape.k)
    W = mi.make_expert_weights(shape, 4, seed=0, experts=np.unique(ids))
    U = len(np.unique(ids))
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        oracle.layer(xb, layer0["Wr_np"], layer0["bias_np"], W, shape.k, layer0["table_np"], shape.E, rb)
        sec = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, old)
    return dict(value=round(T / sec, 3), unit="tokens/s", cores=1, kind="oracle",
                sample=f"one full layer step of weight set 0: T={T} tokens, {T * shape.k} routed rows, "
                       f"{U} experts, single-threaded C oracle (double accumulation) pinned to core {core}, "
                       f"{sec:.2f} s",
                seconds=round(sec, 3), weight_GBps=round(U * shape.bytes_per_expert(4) / sec / 1e9, 4),
                host_cpus=os.cpu_count(), cpu_model=cpu_model())


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.copy_calib_mib or 256)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU expert-parallel design is described, not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi
    import quantized_expert_ffn_gemv_amd as moe

    torch.cuda.set_device(0)
    moe.lib()
    shape = mi.CONFIGS["a3b"]
    bits = 4
    algo = {"auto": moe.ALGO_AUTO, "gemv": moe.ALGO_GEMV, "mfma": moe.ALGO_MFMA}[args.algo]
    log(f"[bench] uploading {args.layers} weight sets of {shape.E * shape.bytes_per_expert(bits) / 1e6:.0f} MB")
    layers = [upload_layer(shape, bits, seed=li, torch=torch, mi=mi, moe=moe) for li in range(args.layers)]
    torch.cuda.synchronize()

    per_expert = shape.bytes_per_expert(bits)
    gate_bytes_per_expert = per_expert * 2 // 3
    down_bytes_per_expert = per_expert // 3
    router_bytes = shape.E * shape.H * 4

    fused = args.ffn == "fused" and "fused" in FFN_KERNELS[args.algo]

    def measure(T, steps, warmup, layer_sets=None):
        r = Runner(torch, mi, moe, shape, layer_sets or layers, T, algo, fused_ffn=fused)
        U = r.experts_used()
        # throughput: the K steps back to back, nothing recorded between kernels
        # (eager calls; with --launch graph, replays of captured graphs)
        eager_ms, eager_wall, _, _ = r.timed(steps, warmup, with_events=False)
        if args.launch == "graph":
            r.capture()
            total_ms, wall = r.timed_graphs(steps, warmup)
        else:
            total_ms, wall = eager_ms, eager_wall
        # kernel durations: the same K steps again with HIP events around the
        # FFN launches on their stream (events between kernels lengthen the
        # step a little, so these passes do not set the throughput); the
        # two-launch FFN is timed too, for its halves
        ev_total_ms, _, ffn_ms, _ = r.timed(steps, 0)
        ffn_launch_us = r.timed_ffn_launches(steps, warmup) if fused else None
        r.fused_ffn = False
        split_total_ms, _, gate_ms, down_ms = r.timed(steps, 2)
        r.fused_ffn = fused
        Us = [U[i % len(U)] for i in range(steps)]
        gate_bytes = sum(u * gate_bytes_per_expert for u in Us)
        down_bytes = sum(u * down_bytes_per_expert for u in Us)
        gate_s, down_s, ffn_s = sum(gate_ms) / 1e3, sum(down_ms) / 1e3, sum(ffn_ms) / 1e3
        if not fused:
            ffn_s = gate_s + down_s
        ms_step = total_ms / steps
        return dict(T=T, steps=steps, ms_per_step=ms_step, tokens_per_s=T * steps / (total_ms / 1e3),
                    eager_ms_per_step=eager_ms / steps,
                    ms_per_step_with_kernel_events=ev_total_ms / steps,
                    split_ms_per_step_with_kernel_events=split_total_ms / steps,
                    wall_s=wall, U_mean=float(np.mean(U)), U_per_set=U,
                    ffn_us=ffn_s / steps * 1e6, gateup_us=gate_s / steps * 1e6, down_us=down_s / steps * 1e6,
                    gateup_GBps=gate_bytes / gate_s / 1e9, down_GBps=down_bytes / down_s / 1e9,
                    ffn_GBps=(gate_bytes + down_bytes) / ffn_s / 1e9,
                    split_ffn_GBps=(gate_bytes + down_bytes) / (gate_s + down_s) / 1e9,
                    layer_GBps=(sum(Us) * per_expert + steps * router_bytes) / (total_ms / 1e3) / 1e9,
                    gateup_bytes_per_launch=gate_bytes / steps,
                    ffn_bytes_per_launch=(gate_bytes + down_bytes) / steps,
                    ffn_launch_us=ffn_launch_us)

    log(f"[bench] T={args.tokens}: {args.warmup} warmup + {args.steps} timed steps")
    main_run = measure(args.tokens, args.steps, args.warmup)
    log(f"[bench] {main_run['tokens_per_s']:.0f} tokens/s, FFN {main_run['ffn_GBps']:.0f} GB/s "
        f"(two launches: gate/up {main_run['gateup_GBps']:.0f}, down {main_run['down_GBps']:.0f} GB/s)")

    sweep = []
    for tok in [int(t) for t in args.sweep.split(",") if t.strip() and t.strip() != "none"]:
        if tok == args.tokens:
            continue
        m = measure(tok, max(args.steps // 2, 10), max(args.warmup // 2, 2))
        log(f"[bench] sweep T={tok}: {m['tokens_per_s']:.0f} tokens/s, FFN {m['ffn_GBps']:.0f} GB/s")
        sweep.append({k: (round(v, 3) if isinstance(v, float) else v) for k, v in m.items()})

    # warm: one weight set only, so the experts a step touches (about 93 MB at
    # T = 32) can stay in the 256 MB last-level cache between steps
    warm = measure(args.tokens, max(args.steps // 2, 10), max(args.warmup // 2, 2), layer_sets=layers[:1])
    log(f"[bench] warm (one weight set) T={args.tokens}: {warm['tokens_per_s']:.0f} tokens/s")

    shared_run = None
    if not args.no_shared_expert:
        # the same step with an always-on shared expert (routed experts' size):
        # its FFN launch first, its sigmoid gate fused into the combine
        shared_sets = [L["shared"] for L in layers]
        n_sh = max(args.steps // 2, 10)
        shared_run = dict(I_shared=shared_sets[0].I, shared_weight_bytes=shape.bytes_per_expert(bits),
                          note="sigmoid gate fused into the combine; one_launch: the shared expert's tiles are "
                               "extra entries of the routed FFN launch; own_launch: a one-expert FFN launch "
                               "before the routing")
        for key, one in (("one_launch", True), ("own_launch", False)):
            rs = Runner(torch, mi, moe, shape, layers, args.tokens, algo, fused_ffn=fused, shared=shared_sets,
                        one_launch=one)
            rs.experts_used()
            sh_ms, _, _, _ = rs.timed(n_sh, max(args.warmup // 2, 2), with_events=False)
            shared_run[key] = dict(tokens_per_s=round(args.tokens * n_sh / (sh_ms / 1e3), 1),
                                   ms_per_step=round(sh_ms / n_sh, 5),
                                   added_us_per_step=round((sh_ms / n_sh - main_run["ms_per_step"]) * 1e3, 2))
            log(f"[bench] with a shared expert ({key}) T={args.tokens}: {shared_run[key]['tokens_per_s']:.0f} "
                f"tokens/s (+{shared_run[key]['added_us_per_step']} us per step)")
            del rs

    # speculative verify ("Strata" page, sec. 3.4): the same T as n_seq sequences of
    # 4 draft tokens whose hidden states correlate, so drafts share expert fetches
    spec_run = None
    if args.tokens % 4 == 0:
        n_seq = args.tokens // 4
        rsv = Runner(torch, mi, moe, shape, layers, args.tokens, algo, fused_ffn=fused,
                     acts=lambda li: mi.make_spec_verify_activations(shape.H, n_seq, 4, seed=2000 + li))
        U_sv = rsv.experts_used()
        n_sv = max(args.steps // 2, 10)
        sv_ms, _, _, _ = rsv.timed(n_sv, max(args.warmup // 2, 2), with_events=False)
        spec_run = dict(sequences=n_seq, drafts_per_sequence=4, rho=0.8,
                        tokens_per_s=round(args.tokens * n_sv / (sv_ms / 1e3), 1), ms_per_step=round(sv_ms / n_sv, 5),
                        experts_used_mean=float(np.mean(U_sv)),
                        experts_used_mean_independent_tokens=main_run["U_mean"])
        log(f"[bench] speculative verify {n_seq} x 4: {spec_run['tokens_per_s']:.0f} tokens/s, "
            f"{spec_run['experts_used_mean']:.1f} experts per step (independent tokens: {main_run['U_mean']:.1f})")
        del rsv

    prefill = None
    if args.prefill_steps > 0:
        prefill = measure_prefill(torch, mi, moe, args.prefill_steps, 3)
        log(f"[bench] prefill: {prefill['tokens_per_s']:.0f} tokens/s, FFN {prefill['ffn_tflops']} TFLOP/s "
            f"({100 * prefill['mfma_util']:.1f}% of bf16 MFMA peak)")

    if fused:
        # the FFN launches timed back to back (events only at the ends): the
        # kernel's own average; the per-step event figure, which also holds the
        # dispatch gap an event between kernels adds, is reported beside it
        achieved = main_run["ffn_bytes_per_launch"] / (main_run["ffn_launch_us"] * 1e-6) / 1e9
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic_record(args.algo, "fused"),
                        kernel=FFN_KERNELS[args.algo]["fused"] + " (gate/up matvec + SwiGLU + down matvec, one launch)",
                        algorithmic_bytes_per_launch=round(main_run["ffn_bytes_per_launch"]),
                        mean_launch_us=round(main_run["ffn_launch_us"], 3),
                        launches_timed=args.steps,
                        in_step_event_us=round(main_run["ffn_us"], 3))
    else:
        achieved = main_run["gateup_GBps"]
        roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic_record(args.algo, "gateup"),
                        kernel=FFN_KERNELS[args.algo]["gateup"] + " (gate/up matvec + SwiGLU)",
                        algorithmic_bytes_per_launch=round(main_run["gateup_bytes_per_launch"]),
                        mean_launch_us=round(main_run["gateup_us"], 3))

    if args.copy_calib_mib:
        n = args.copy_calib_mib * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one step")
        cpu = cpu_baseline(mi, shape, layers[0], args.tokens)

    result = {
        "metric": "MoE-layer decode tokens/s + weight-stream HBM GB/s (% of MI355X peak)",
        "value": round(main_run["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"A3B-style MoE decode layer, T={args.tokens} tokens: hidden 2048, 256 experts top-8 "
                        f"(renormalised gates), intermediate 512, SwiGLU, 4-bit g128 weights "
                        f"(fp16 scale+bias), bf16 activations, Zipf(1.1) routing, "
                        f"{shape.n_resident}/256 resident, {args.layers} rotating weight sets",
            "H": shape.H, "E": shape.E, "k": shape.k, "I": shape.I, "T": args.tokens, "bits": bits,
            "group": 128, "weight_sets": args.layers, "algo": args.algo, "ffn": "fused" if fused else "split",
            "launch": "one HIP graph per layer step, replayed" if args.launch == "graph" else "eager calls",
            "parallelism": "none (one GPU)",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "weight_stream": {
            "experts_used_mean": main_run["U_mean"],
            "ffn_GBps": round(main_run["ffn_GBps"], 1),
            "ffn_frac_of_peak": round(main_run["ffn_GBps"] / HBM_PEAK_GBPS, 4),
            "ffn_us": round(main_run["ffn_us"], 3),
            "layer_GBps_incl_router": round(main_run["layer_GBps"], 1),
            "ms_per_step_with_kernel_events": round(main_run["ms_per_step_with_kernel_events"], 5),
            "eager_ms_per_step": round(main_run["eager_ms_per_step"], 5),
            "two_launch_gateup_GBps": round(main_run["gateup_GBps"], 1),
            "two_launch_down_GBps": round(main_run["down_GBps"], 1),
            "two_launch_ffn_GBps": round(main_run["split_ffn_GBps"], 1),
            "two_launch_gateup_us": round(main_run["gateup_us"], 3),
            "two_launch_down_us": round(main_run["down_us"], 3),
            "two_launch_ms_per_step_with_kernel_events": round(main_run["split_ms_per_step_with_kernel_events"], 5),
        },
        "sweep": sweep,
        "warm_one_weight_set": {"tokens_per_s": round(warm["tokens_per_s"], 1),
                                "ms_per_step": round(warm["ms_per_step"], 5),
                                "ffn_GBps": round(warm["ffn_GBps"], 1)},
        "shared_expert": shared_run,
        "spec_verify": spec_run,
        "prefill": prefill,
        "context_not_comparable": CONTEXT,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
