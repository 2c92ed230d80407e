"""The non-default workloads of bench.py (``--workload projections|prefill|sharded``).

Each prints one JSON line in the same format as the default decode run:

* projections -- the replicated attention-projection layer: 8 FP8 projections
  ([24576x7168], [8192x7168], [7168x8192], [4096x7168], [1000x7168],
  [7168x3072], [3072x7168], [1536x7168], 385.2 MB per layer), 16 layers, N=16
  chunks, M=16 tokens.  One step = one pipelined forward (side-stream
  reassembly of layer l+1 while the 8 projections of layer l run through
  views of the other slot).  Metric: weight-stream GB/s.
* prefill -- the shared-expert MLP (hidden 6144, intermediate 14336, FP8
  weights, BF16 activations) at M = 4096 and 16384 tokens, 4 layers, N=16,
  the reassembly overlapped on the side stream.  Metric: TFLOP/s
  (6*M*H*I per layer) against the dense BF16 matrix-core peak.
* sharded -- X[2048x8192] @ W[8192x28672] in BF16 computed as the full
  product, as 8 output-column shards written into their slices of Y, and as
  8 contraction shards whose fp32 partials are summed in shard order.
  Metric: TFLOP/s over the three variants.

Inputs are the seeded synthetic ones of ``synth``.  The timed region holds
only device work on resident inputs; durations of the dominant kernel come
from HIP events on the stream it runs on.
"""
from __future__ import annotations

import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0    # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK = 2500.0   # TFLOP/s, dense BF16 matrix cores (no sparsity)
MFMA_FP8_PEAK = 5000.0    # TFLOP/s, dense FP8 matrix cores (no sparsity)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


class FenceFreeEvents:
    """HIP timing events without the system-scope fence on record (the kind the
    planner's timing uses), made through the HIP runtime torch has loaded."""

    def __init__(self, n: int):
        import ctypes

        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(0x20000000))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i: int, stream) -> None:
        rc = self._hip.hipEventRecord(self.ev[i], self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self) -> None:
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def _pack_layers(swr, torch, dev, wl, n_layers):
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, wl.n_chunks)
    chunks, scales = [], []
    for layer in range(n_layers):
        ws = wl.layer_weights(layer)
        src = [torch.from_numpy(w.raw()).to(dev) for w in ws]
        cl = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=dev) for _ in range(wl.n_chunks)]
        swr.pack_layer(lay, views, src, cl)
        torch.cuda.synchronize()
        del src
        chunks.append(cl)
        scales.append([torch.from_numpy(w.scale).to(dev) if w.scale is not None else None for w in ws])
        log(f"layer {layer} packed into {wl.n_chunks} chunks of {lay['chunk_bytes']} B")
    return views, lay, chunks, scales


GATES = ("done", "begin", "after")


class _Pipeline:
    """A planner over ping-pong slots plus the timing the report needs.
    gate: "done" (the pages' gate), "begin" or "after"; queues: 2 puts the
    gathers on a side stream, 1 on the compute stream itself."""

    def __init__(self, swr, torch, dev, lay, chunks, gate="done", queues=2):
        self.swr, self.torch = swr, torch
        T, C = lay["total_bytes"], lay["chunk_bytes"]
        self.L = len(chunks)
        self.slot_a = torch.empty(T, dtype=torch.uint8, device=dev)
        self.slot_b = torch.empty(T, dtype=torch.uint8, device=dev)
        self.compute = torch.cuda.Stream()
        self.side_stream = torch.cuda.Stream()
        self.chunks, self.C = chunks, C
        self.gate, self.queues = gate, queues
        self.planner = self.make_planner(gate, queues)

    def make_planner(self, gate, queues):
        swr = self.swr
        p = swr.Planner(0, self.L, self.compute, self.compute if queues == 1 else self.side_stream, self.slot_a,
                        self.slot_b)
        for layer in range(self.L):
            p.set_layer(layer, self.chunks[layer], self.C)
        if self.L % 2 == 0:
            p.set_cyclic(True)
        p.set_gate({"done": swr.GATE_DONE, "begin": swr.GATE_BEGIN, "after": swr.GATE_AFTER}[gate])
        return p

    def forward(self, layer_fn, planner=None):
        p = self.planner if planner is None else planner
        p.reset()
        p.pre_dispatch(0)
        for layer in range(self.L):
            p.maybe_dispatch(layer + 1)
            base = p.wait_ready_once(layer)
            layer_fn(layer, base)
            p.update_done_event(layer)

    def serial_forward(self, layer_fn, events=None, inner=True):
        inner = events is not None and inner
        if events is not None:
            events.record(4 * self.L, self.compute)
        for layer in range(self.L):
            s = self.slot_a if layer % 2 == 0 else self.slot_b
            if inner:
                events.record(4 * layer, self.compute)
            self.swr.reassemble_into_slot(self.chunks[layer], self.C, s, stream=self.compute)
            if inner:
                events.record(4 * layer + 1, self.compute)
                events.record(4 * layer + 2, self.compute)
            layer_fn(layer, s.data_ptr())
            if inner:
                events.record(4 * layer + 3, self.compute)
        if events is not None:
            events.record(4 * self.L + 1, self.compute)

    def timed(self, layer_fn, steps, warmup, every=1):
        """Pipelined forwards: (wall s, per-forward ms, per-layer compute ms, gather ms).
        The planner's own fence-free timing events time each gather on the
        stream it runs on and each layer's compute from its begin (after the
        ready wait) to its done record, in every `every`-th step (the
        forwards of the other steps carry only their own two events)."""
        torch = self.torch
        with torch.cuda.stream(self.compute):
            for _ in range(warmup):
                self.forward(layer_fn)
        torch.cuda.synchronize()
        fwd = FenceFreeEvents(2 * steps)
        self.sampled = [s for s in range(steps) if s % max(1, every) == 0]
        self.planner.set_timing(len(self.sampled) * self.L)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.compute):
            for s in range(steps):
                self.planner.pause_timing(s not in self.sampled)
                fwd.record(2 * s, self.compute)
                self.forward(layer_fn)
                fwd.record(2 * s + 1, self.compute)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gathers = self.planner.gather_times()
        layer_ms = self.planner.layer_times()
        self.planner.pause_timing(False)
        self.planner.set_timing(0)
        fwd_ms = [fwd.elapsed_ms(2 * s, 2 * s + 1) for s in range(steps)]
        fwd.close()
        return wall, fwd_ms, layer_ms, gathers

    def timed_bare(self, layer_fn, reps, planner=None):
        """ms per pipelined forward with no timing events between kernels."""
        torch = self.torch
        with torch.cuda.stream(self.compute):
            self.forward(layer_fn, planner)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.compute)
            for _ in range(reps):
                self.forward(layer_fn, planner)
            e1.record(self.compute)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def schedules(self, layer_fn, reps):
        """ms per forward without timing events for each gate on two queues
        and the done/after gates on one queue."""
        out = {}
        for gate, q in [(g, 2) for g in GATES] + [("done", 1), ("after", 1)]:
            p = self.make_planner(gate, q)
            out[f"gate_{gate}_queues_{q}"] = round(self.timed_bare(layer_fn, reps, p), 4)
            p.close()
        return out

    def timed_serial(self, layer_fn, reps, level=0):
        """The same gathers and layers back to back on the compute stream;
        level 1: the forward bracketed by two fence-free events, as the timed
        steps' forwards are; level 2: also around each gather and each layer,
        as in the steps the planner times."""
        torch = self.torch
        ev = FenceFreeEvents(4 * self.L + 2) if level else None
        with torch.cuda.stream(self.compute):
            self.serial_forward(layer_fn, ev, level > 1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.compute)
            for _ in range(reps):
                self.serial_forward(layer_fn, ev, level > 1)
            e1.record(self.compute)
        torch.cuda.synchronize()
        if ev is not None:
            ev.close()
        return e0.elapsed_time(e1) / reps

    def bare_trials(self, layer_fn, reps, trials=3):
        """Serial and default-schedule forwards without timing events, timed in
        alternating trials: (median serial ms, median pipelined ms, trials)."""
        import numpy as np

        ts, tp = [], []
        for _ in range(trials):
            ts.append(self.timed_serial(layer_fn, reps))
            tp.append(self.timed_bare(layer_fn, reps))
        return float(np.median(ts)), float(np.median(tp)), {"serial": [round(t, 4) for t in ts],
                                                           "pipelined": [round(t, 4) for t in tp]}

    def isolated_gather_ms(self, reps):
        torch = self.torch
        with torch.cuda.stream(self.compute):
            for layer in range(self.L):
                self.swr.reassemble_into_slot(self.chunks[layer], self.C, self.slot_a, stream=self.compute)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.compute)
            for _ in range(reps):
                for layer in range(self.L):
                    s = self.slot_a if layer % 2 == 0 else self.slot_b
                    self.swr.reassemble_into_slot(self.chunks[layer], self.C, s, stream=self.compute)
            e1.record(self.compute)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * self.L)

    def close(self):
        self.planner.close()


def _isolated(torch, stream, fn, n_layers, reps):
    """ms per layer of fn(layer) run back to back on `stream`."""
    with torch.cuda.stream(stream):
        for layer in range(n_layers):
            fn(layer)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for layer in range(n_layers):
                fn(layer)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n_layers)


def _base_record(args, metric, value, unit, ms_per_step, dtype, data, config, higher=True):
    return {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": higher,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": data, "config": config,
    }


# ----------------------------------------------------------------------------- projections
def run_projections(args, swr, torch, np, synth, dev):
    wl = synth.ATTN_PROJECTIONS
    L = args.layers or wl.layers
    m = wl.tokens[0]
    views, lay, chunks, scales = _pack_layers(swr, torch, dev, wl, L)
    T = lay["total_bytes"]
    w_bytes = sum(v["nbytes"] for v in views)
    s_bytes = sum(o * 4 for _, o, _, _ in wl.weights)
    in_dims = []
    for _, _, i, _ in wl.weights:
        if i not in in_dims:
            in_dims.append(i)
    xs = {i: torch.from_numpy(synth.activations(synth.seed_for(3, 0, 50 + j), m, i).view(np.int16).copy())
          .view(torch.bfloat16).to(dev) for j, i in enumerate(in_dims)}
    ys = [torch.empty((m, o), dtype=torch.bfloat16, device=dev) for _, o, _, _ in wl.weights]
    # decode-shaped (16 tokens): the gather and the projections both stream
    # HBM, so the default is the one-GPU schedule (gate after, one queue)
    pipe = _Pipeline(swr, torch, dev, lay, chunks, gate=args.gate, queues=args.queues)

    def projs(layer, base):
        return [dict(w=base + views[j]["offset"], dtype=d, row_scale=scales[layer][j], out_f=o, in_f=i, x=xs[i],
                     y=ys[j]) for j, (_, o, i, d) in enumerate(wl.weights)]

    # all 8 projections of a layer in one grouped launch (no scratch needed when they stage)
    wsz = swr.proj_grouped_workspace_bytes(projs(0, chunks[0][0].data_ptr()), m)
    wsp = torch.empty(wsz, dtype=torch.uint8, device=dev) if wsz > 0 else None

    def layer_fn(layer, base):
        swr.proj_forward_grouped(projs(layer, base), m, workspace=wsp, stream=pipe.compute)

    wall, fwd_ms, layer_ms, gathers = pipe.timed(layer_fn, args.steps, args.warmup, every=args.timing_every)
    sampled = pipe.sampled
    full = [torch.empty(T, dtype=torch.uint8, device=dev) for _ in range(L)]
    for layer in range(L):
        swr.reassemble_into_slot(chunks[layer], lay["chunk_bytes"], full[layer], stream=pipe.compute)
    torch.cuda.synchronize()
    iso = _isolated(torch, pipe.compute, lambda layer: layer_fn(layer, full[layer].data_ptr()), L,
                    args.isolated_reps)
    del full
    iso_gather = pipe.isolated_gather_ms(args.isolated_reps)
    serial_timed = pipe.timed_serial(layer_fn, args.isolated_reps, level=2)
    serial = pipe.timed_serial(layer_fn, args.isolated_reps, level=1)
    serial_bare, pipelined_bare, trials = pipe.bare_trials(layer_fn, max(4, args.steps // 2))
    schedules = pipe.schedules(layer_fn, max(4, args.steps // 2))
    pipe.close()

    alg = w_bytes + s_bytes + sum(m * i * 2 for _, _, i, _ in wl.weights) + sum(m * o * 2 for _, o, _, _ in wl.weights)
    layer_avg = float(np.mean(layer_ms))
    gather_avg = float(np.mean(gathers))
    value = L * args.steps * (w_bytes + s_bytes) / wall / 1e9
    # forwards without the planner's timing records, and the sampled ones
    # that carry them; means, like the serial references'
    plain = [t for s, t in enumerate(fwd_ms) if s not in sampled]
    fwd = float(np.mean(plain if plain else fwd_ms))
    fwd_timed = float(np.mean([fwd_ms[s] for s in sampled]))
    kernels = {
        "projection_layer": {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS, "bytes_per_launch": alg,
                             "avg_ms": layer_avg, "achieved": alg / (layer_avg * 1e-3) / 1e9},
        "reassemble_into_slot": {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS, "bytes_per_launch": 2 * T,
                                 "avg_ms": gather_avg, "achieved": 2 * T / (gather_avg * 1e-3) / 1e9},
    }
    for k in kernels.values():
        k["frac"] = k["achieved"] / k["peak"]
        k["traffic"] = None
    dom = "projection_layer" if sum(layer_ms) >= sum(gathers) else "reassemble_into_slot"
    dk = kernels[dom]

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gemm

        w = wl.layer_weights(0)[1]  # [8192 x 7168]
        x = synth.activations(synth.seed_for(3, 0, 50), m, w.in_features)
        t = time.perf_counter()
        gemm.proj(x, w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        dt = time.perf_counter() - t
        cpu = {"value": round((w.nbytes + 4 * w.out_features) / dt / 1e9, 3), "unit": "GB/s", "cores": _threads(),
               "kind": "oracle", "sample": f"one [{w.out_features}x{w.in_features}] FP8 projection at M={m}, "
                                           "float64 NumPy oracle, one run"}

    rec = _base_record(args, "replicated projection weight-stream GB/s at M=16", value, "GB/s",
                       wall * 1e3 / args.steps, "fp8_e4m3fn weights x bf16 activations, fp32 accumulate",
                       "synthetic: seeded N(0,0.02) weights quantised per row to E4M3FN, N(0,1) bf16 tokens",
                       {"workload": wl.name, "layers": L, "n_chunks": wl.n_chunks, "tokens": m, "layer_bytes": T,
                        "projections": [[o, i] for _, o, i, _ in wl.weights],
                        "gate": args.gate, "queues": args.queues,
                        "step": "pipelined forward (reassembly + the 8 projections as one grouped launch, per "
                                "layer through the planner) over all layers"})
    rec.update({
        "value_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "pipelined_ms_per_forward": round(fwd, 4),
        "isolated_layer_ms": round(iso, 4),
        "isolated_weight_GBps": round((w_bytes + s_bytes) / (iso * 1e-3) / 1e9, 1),
        "isolated_weight_frac": round((w_bytes + s_bytes) / (iso * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "isolated_reassembly_GBps": round(2 * T / (iso_gather * 1e-3) / 1e9, 1),
        "serial_reference_ms_per_forward": round(serial, 4),
        "pipelined_timed_ms_per_forward": round(fwd_timed, 4),
        "serial_reference_timed_ms_per_forward": round(serial_timed, 4),
        "serial_reference_bare_ms_per_forward": round(serial_bare, 4),
        "pipelined_bare_ms_per_forward": round(pipelined_bare, 4),
        "bare_trials_ms_per_forward": trials,
        "schedules_ms_per_forward": schedules,
        "compute_stall_ms": round(fwd - L * layer_avg, 4),
        "gather_to_compute_ratio": round(gather_avg / layer_avg, 3),
        "exposed_ms_per_layer": round(fwd / L - layer_avg, 4),
        "roofline": {"bound": dk["bound"], "achieved": round(dk["achieved"], 1), "peak": dk["peak"],
                     "unit": dk["unit"], "frac": round(dk["frac"], 4), "traffic": None, "kernel": dom},
        "roofline_by_kernel": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                               for k, v in kernels.items()},
        "cpu_baseline": cpu,
    })
    return rec


# ----------------------------------------------------------------------------- prefill
def run_prefill(args, swr, torch, np, synth, dev):
    wl = synth.SHARED_EXPERT_PREFILL
    L = args.layers or wl.layers
    H, I = wl.hidden, wl.intermediate
    tokens = [int(t) for t in args.tokens.split(",")] if args.tokens != "1,8,32,64" else wl.tokens
    views, lay, chunks, scales = _pack_layers(swr, torch, dev, wl, L)
    T = lay["total_bytes"]
    o_gu, o_d = views[0]["offset"], views[1]["offset"]
    pipe = _Pipeline(swr, torch, dev, lay, chunks)
    per_m, total_flops, total_wall, dom_ms, dom_flops = {}, 0.0, 0.0, [], 0.0
    gather_all = []
    for m in tokens:
        x = torch.from_numpy(synth.activations(synth.seed_for(4, 0, 50), m, H).view(np.int16).copy()) \
            .view(torch.bfloat16).to(dev)
        y = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(swr.mlp_workspace_bytes(m, H, I, "fp8_e4m3fn"), dtype=torch.uint8, device=dev)

        def layer_fn(layer, base, x=x, y=y, ws=ws):
            swr.mlp_forward(base + o_gu, scales[layer][0], base + o_d, scales[layer][1], "fp8_e4m3fn", H, I, x, y, ws,
                            stream=pipe.compute)

        wall, fwd_ms, layer_ms, gathers = pipe.timed(layer_fn, args.steps, args.warmup)
        gather_all += gathers
        flops = 6.0 * m * H * I
        layer_avg = float(np.mean(layer_ms))
        fwd = float(np.median(fwd_ms))
        total_flops += flops * L * args.steps
        total_wall += wall
        dom_ms += layer_ms
        dom_flops += flops * len(layer_ms)
        per_m[str(m)] = {
            "pipelined_ms_per_forward": round(fwd, 4),
            "pipelined_TFLOPs": round(flops * L / (fwd * 1e-3) / 1e12, 1),
            "mlp_ms_per_layer_in_pipeline": round(layer_avg, 4),
            "mlp_TFLOPs_in_pipeline": round(flops / (layer_avg * 1e-3) / 1e12, 1),
            "mfma_bf16_frac": round(flops / (layer_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK, 4),
            "compute_stall_ms": round(fwd - L * layer_avg, 4),
            "gather_ms_avg": round(float(np.mean(gathers)), 4),
            "tokens_per_s": round(m * args.steps / wall, 1),
        }
        del x, y, ws

    # The same pipelined forwards with FP8 activations (swr_mlp_forward_fp8act:
    # X and h quantised per token, FP8 x FP8 matrix cores), an option beyond
    # the pages' BF16 activations; reported beside the headline.
    fp8act = {}
    for m in tokens:
        x = torch.from_numpy(synth.activations(synth.seed_for(4, 0, 50), m, H).view(np.int16).copy()) \
            .view(torch.bfloat16).to(dev)
        y = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(swr.mlp_fp8act_workspace_bytes(m, H, I), dtype=torch.uint8, device=dev)

        def layer_fn8(layer, base, x=x, y=y, ws=ws):
            swr.mlp_forward_fp8act(base + o_gu, scales[layer][0], base + o_d, scales[layer][1], H, I, x, y, ws,
                                   stream=pipe.compute)

        wall, fwd_ms, layer_ms, gathers = pipe.timed(layer_fn8, args.steps, args.warmup)
        flops = 6.0 * m * H * I
        layer_avg = float(np.mean(layer_ms))
        fwd = float(np.median(fwd_ms))
        fp8act[str(m)] = {
            "pipelined_ms_per_forward": round(fwd, 4),
            "pipelined_TFLOPs": round(flops * L / (fwd * 1e-3) / 1e12, 1),
            "mlp_ms_per_layer_in_pipeline": round(layer_avg, 4),
            "mlp_TFLOPs_in_pipeline": round(flops / (layer_avg * 1e-3) / 1e12, 1),
            "mfma_fp8_frac": round(flops / (layer_avg * 1e-3) / 1e12 / MFMA_FP8_PEAK, 4),
            "tokens_per_s": round(m * args.steps / wall, 1),
        }
        del x, y, ws
    pipe.close()
    value = total_flops / total_wall / 1e12
    achieved = dom_flops / (sum(dom_ms) * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gemm

        gu, d = wl.layer_weights(0)
        xs = synth.activations(synth.seed_for(4, 0, 50), 8, H)
        t = time.perf_counter()
        gemm.mlp(xs, gu.raw(), gu.scale, d.raw(), d.scale, gu.dtype, H, I)
        dt = time.perf_counter() - t
        cpu = {"value": round(6.0 * 8 * H * I / dt / 1e9, 3), "unit": "GFLOP/s", "cores": _threads(),
               "kind": "oracle", "sample": "8 tokens through one shared-expert layer (the oracle's cost is the FP8 "
                                           "decode plus a float64 product per token row), one run"}

    rec = _base_record(args, "prefill MLP TFLOP/s (fraction of the dense BF16 matrix-core peak)", value, "TFLOP/s",
                       total_wall * 1e3 / args.steps, "fp8_e4m3fn weights widened to bf16, bf16 MFMA, fp32 accumulate",
                       "synthetic: seeded N(0,0.02) weights quantised per row to E4M3FN, N(0,1) bf16 tokens",
                       {"workload": wl.name, "hidden": H, "intermediate": I, "layers": L, "n_chunks": wl.n_chunks,
                        "tokens": tokens, "layer_bytes": T,
                        "step": "pipelined forward (side-stream reassembly + MLP) over all layers for every M"})
    rec.update({
        "value_frac_of_mfma_bf16_peak": round(value / MFMA_BF16_PEAK, 4),
        "per_tokens": per_m,
        "reassembly_ms_avg_in_pipeline": round(float(np.mean(gather_all)), 4),
        "fp8_activations": fp8act,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK, 4), "traffic": None, "kernel": "mlp_forward"},
        "cpu_baseline": cpu,
    })
    return rec


# ----------------------------------------------------------------------------- sharded matmul
def run_sharded(args, swr, torch, np, synth, dev):
    wl = synth.SHARDED_MATMUL
    B, D, F, S = wl.extra["B"], wl.extra["D"], wl.extra["F"], wl.extra["shards"]
    x_bits, w_t_bits = synth.sharded_matmul_inputs(B, D, F)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w_t = torch.from_numpy(w_t_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    fs, ds = F // S, D // S
    # contraction shards as a rank would hold them: X[:, jD/S:(j+1)D/S] and W^T[:, same], contiguous
    xk = [x[:, j * ds:(j + 1) * ds].contiguous() for j in range(S)]
    wk = [w_t[:, j * ds:(j + 1) * ds].contiguous() for j in range(S)]
    y_full = torch.empty((B, F), dtype=torch.bfloat16, device=dev)
    y_cols = torch.empty((B, F), dtype=torch.bfloat16, device=dev)
    y_k = torch.empty((B, F), dtype=torch.bfloat16, device=dev)
    parts = [torch.empty((B, F), dtype=torch.float32, device=dev) for _ in range(S)]
    stream = torch.cuda.Stream()
    esz = 2

    def full():
        swr.proj_forward(w_t, "bf16", None, F, D, x, y_full, stream=stream)

    # the S shard GEMMs of a variant go in one grouped call (one launch over all
    # their tiles: a single shard fills less than one wave of the CUs)
    col_projs = [dict(w=w_t.data_ptr() + j * fs * D * esz, dtype="bf16", row_scale=None, out_f=fs, in_f=D, x=x,
                      y=y_cols.data_ptr() + j * fs * esz, ldy=F, y_fp32=False) for j in range(S)]
    k_projs = [dict(w=wk[j], dtype="bf16", row_scale=None, out_f=F, in_f=ds, x=xk[j], y=parts[j], y_fp32=True)
               for j in range(S)]

    def columns():
        swr.proj_forward_grouped(col_projs, B, stream=stream)

    def kshard_gemms():
        swr.proj_forward_grouped(k_projs, B, stream=stream)

    def kshards():
        kshard_gemms()
        swr.sum_partials(parts, y_k, stream=stream)

    variants = {"full": full, "column_shards": columns, "k_shards_plus_sum": kshards}
    flops = 2.0 * B * D * F
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for fn in variants.values():
                fn()
    torch.cuda.synchronize()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
          for k in variants}
    sum_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for s in range(args.steps):
            for k, fn in variants.items():
                ev[k][s][0].record(stream)
                if k == "k_shards_plus_sum":
                    kshard_gemms()
                    sum_ev[s][0].record(stream)
                    swr.sum_partials(parts, y_k, stream=stream)
                    sum_ev[s][1].record(stream)
                else:
                    fn()
                ev[k][s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: float(np.median([a.elapsed_time(b) for a, b in ev[k]])) for k in variants}
    sum_ms = float(np.median([a.elapsed_time(b) for a, b in sum_ev]))
    col_equal = bool(torch.equal(y_full, y_cols))
    value = 3 * flops * args.steps / wall / 1e12
    sum_bytes = S * B * F * 4 + B * F * 2
    achieved = flops / (ms["full"] * 1e-3) / 1e12
    per = {k: {"ms": round(v, 4), "TFLOPs": round(flops / (v * 1e-3) / 1e12, 1)} for k, v in ms.items()}
    per["k_shards_plus_sum"]["sum_partials_ms"] = round(sum_ms, 4)
    per["k_shards_plus_sum"]["sum_partials_GBps"] = round(sum_bytes / (sum_ms * 1e-3) / 1e9, 1)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gemm

        rows = 16
        t = time.perf_counter()
        gemm.matmul_f64(x_bits[:rows], w_t_bits)
        dt = time.perf_counter() - t
        cpu = {"value": round(2.0 * rows * D * F / dt / 1e9, 3), "unit": "GFLOP/s", "cores": _threads(),
               "kind": "oracle", "sample": f"{rows} rows of X through the full product (float64 NumPy), one run"}

    rec = _base_record(args, "sharded-matmul TFLOP/s (full, column shards, K shards + sum)", value, "TFLOP/s",
                       wall * 1e3 / args.steps, "bf16", "synthetic: seeded N(0,1) X, N(0,0.02) W, bf16",
                       {"workload": wl.name, "B": B, "D": D, "F": F, "shards": S,
                        "step": "the three variants once each"})
    rec.update({
        "variants": per,
        "column_shards_bitwise_equal_full": col_equal,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK, 4), "traffic": None, "kernel": "proj_forward (full)"},
        "roofline_sum_partials": {"bound": "hbm", "achieved": round(sum_bytes / (sum_ms * 1e-3) / 1e9, 1),
                                  "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                  "frac": round(sum_bytes / (sum_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": cpu,
    })
    return rec


def run(args) -> int:
    import numpy as np
    import torch

    import sharded_weight_reassembly_amd as swr
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fn = {"projections": run_projections, "prefill": run_prefill, "sharded": run_sharded}[args.workload]
    rec = fn(args, swr, torch, np, synth, dev)
    print(json.dumps(rec), flush=True)
    return 0
