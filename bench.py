#!/usr/bin/env python3
"""Benchmark of the flat-weight reassembly hot path on one MI355X.

Workload: the shared-expert decode MLP stack -- hidden 6144, intermediate
14336, FP8 E4M3FN weights with fp32 row scales (gate_up [28672 x 6144] =
176.2 MB, down [6144 x 14336] = 88.1 MB per layer), 8 layers, each layer's
flat buffer held as N=16 byte chunks in HBM, two ping-pong slots.

One step = one pipelined forward through the 8 layers for every token count
M in the sweep (1, 8, 32, 64): the planner gathers layer l+1 into a slot on a
side stream (gated by done(l-1)) while the compute stream runs layer l's
gate_up -> SiLU*up -> down through zero-copy views of the other slot.

Printed (one JSON line): `value` is whole-job decode-MLP weight-stream
throughput, i.e. the weight + scale bytes the MLPs consumed during the K
timed steps divided by their wall time (the reassembly traffic shares the
same HBM).  Also: per-M tokens/s, isolated GEMM and reassembly bandwidths,
the roofline of the dominant kernel from HIP-event durations taken during
the timed steps, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
YIELD_LDS = 56 * 1024  # gather LDS reservation reported beside the headline


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=["decode", "projections", "prefill", "sharded"], default="decode",
                    help="decode (default, the headline): shared-expert decode MLP stack; projections: the "
                         "replicated attention-projection layers at M=16; prefill: the shared-expert MLP at "
                         "M=4096/16384; sharded: the sharded-matmul layouts (full, column shards, K shards)")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=str, default="1,8,32,64")
    ap.add_argument("--curve-tokens", type=str, default="2,4,16",
                    help="further token counts timed isolated only, to draw the decode MLP's curve")
    ap.add_argument("--layers", type=int, default=0, help="layers of the workload (0: its own count)")
    ap.add_argument("--gate", choices=["done", "begin", "after"], default="after",
                    help="decode: what the gather of layer l+1 waits for -- layer l-1 being done (the pages' gate), "
                         "the compute stream beginning layer l, or layer l being done (no overlap; the default: "
                         "on one GPU the gather and the GEMMs share one HBM)")
    ap.add_argument("--queues", type=int, choices=[1, 2], default=1,
                    help="decode: 2 puts the gathers on a side stream, 1 on the compute stream itself (one queue)")
    ap.add_argument("--gather-lds", type=int, default=0,
                    help="decode: LDS bytes each copy workgroup of the planner's gathers reserves, to leave CUs "
                         "to the GEMMs (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--minimal", action="store_true",
                    help="only the pipelined steps and isolated kernels (no serial, DMA, tensor-parallel or graph "
                         "sections)")
    ap.add_argument("--isolated-reps", type=int, default=10)
    ap.add_argument("--timing-every", type=int, default=4,
                    help="the planner times the gathers and layers of every k-th timed step (a timing record "
                         "costs about 2 us between two kernels)")
    ap.add_argument("--isolated-only", action="store_true",
                    help="decode: only the isolated MLPs at every M and the isolated gathers, then the calibration "
                         "copy (for hardware-counter runs)")
    ap.add_argument("--timed-only", action="store_true",
                    help="decode: only the warmup and the timed steps (for a kernel trace of the timed region)")
    ap.add_argument("--calibration-copy-mib", type=int, default=256,
                    help="size of a plain device copy run at the end; rocprofv3 --pmc runs use it to scale "
                         "FETCH_SIZE/WRITE_SIZE into bytes")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the reassembly path here is the "
              f"one-GPU share of the method, with all N chunks resident in one HBM; no multi-GPU run exists.",
              file=sys.stderr)
        return 2
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if world != 1:
        print("bench.py must not be launched with more than one rank", file=sys.stderr)
        return 2
    if args.workload != "decode":
        import bench_workloads

        return bench_workloads.run(args)

    import numpy as np
    import torch

    import sharded_weight_reassembly_amd as swr
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tokens = [int(t) for t in args.tokens.split(",")]
    wl = synth.SHARED_EXPERT_DECODE
    H, I, N, L = wl.hidden, wl.intermediate, wl.n_chunks, (args.layers or wl.layers)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, N)
    T, C = lay["total_bytes"], lay["chunk_bytes"]
    w_bytes = sum(v["nbytes"] for v in views)
    s_bytes = (2 * I + H) * 4

    # ---------------------------------------------------------------- setup
    t0 = time.time()
    chunks, scales = [], []
    for layer in range(L):
        ws = wl.layer_weights(layer)
        src = [torch.from_numpy(w.raw()).to(dev) for w in ws]
        cl = [torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(N)]
        swr.pack_layer(lay, views, src, cl)
        torch.cuda.synchronize()
        del src
        chunks.append(cl)
        scales.append([torch.from_numpy(w.scale).to(dev) for w in ws])
        log(f"layer {layer} packed into {N} chunks of {C} B")
    log(f"setup {time.time() - t0:.1f}s")
    slot_a = torch.empty(T, dtype=torch.uint8, device=dev)
    slot_b = torch.empty(T, dtype=torch.uint8, device=dev)
    # the isolated MLPs also run at the curve's token counts (not in
    # --isolated-only, whose counter runs attribute launches by token count)
    curve = [] if args.isolated_only or not args.curve_tokens else [int(t) for t in args.curve_tokens.split(",")]
    iso_tokens = sorted(set(tokens) | set(curve))
    x_all = synth.activations(synth.seed_for(2, 0, 50), max(iso_tokens), H)
    xs = {m: torch.from_numpy(x_all[:m].view(np.int16).copy()).view(torch.bfloat16).to(dev) for m in iso_tokens}
    ys = {m: torch.empty((m, H), dtype=torch.bfloat16, device=dev) for m in iso_tokens}
    wsp = {m: torch.empty(swr.mlp_workspace_bytes(m, H, I, "fp8_e4m3fn"), dtype=torch.uint8, device=dev)
           for m in iso_tokens}

    compute = torch.cuda.Stream()
    side_stream = torch.cuda.Stream()
    side = compute if args.queues == 1 else side_stream
    gate_of = {"begin": swr.GATE_BEGIN, "done": swr.GATE_DONE, "after": swr.GATE_AFTER}

    def make_planner(gate: str, queues: int, gather_lds: int = 0, cyclic: bool = True):
        pl = swr.Planner(0, L, compute, compute if queues == 1 else side_stream, slot_a, slot_b)
        for layer in range(L):
            pl.set_layer(layer, chunks[layer], C)
        if cyclic and L % 2 == 0:
            # forwards run back to back: each gathers the next one's first layer during its last layer
            pl.set_cyclic(True)
        pl.set_gate(gate_of[gate])
        pl.set_gather_lds(gather_lds)
        return pl

    planner = make_planner(args.gate, args.queues, args.gather_lds)
    o_gu, o_d = views[0]["offset"], views[1]["offset"]

    def forward(m: int, gemm_events=None, pl=None) -> None:
        pl = planner if pl is None else pl
        pl.reset()
        pl.pre_dispatch(0)
        for layer in range(L):
            pl.maybe_dispatch(layer + 1)
            base = pl.wait_ready_once(layer)
            if gemm_events is not None:
                gemm_events[layer][0].record(compute)
            swr.mlp_forward(base + o_gu, scales[layer][0], base + o_d, scales[layer][1], "fp8_e4m3fn", H, I, xs[m],
                            ys[m], wsp[m], stream=compute)
            if gemm_events is not None:
                gemm_events[layer][1].record(compute)
            pl.update_done_event(layer)

    # ---------------------------------------------------------------- isolated kernels
    # every layer reassembled into its own buffer, then the MLPs alone and the gathers alone
    def isolated_kernels():
        full = [torch.empty(T, dtype=torch.uint8, device=dev) for _ in range(L)]
        for layer in range(L):
            swr.reassemble_into_slot(chunks[layer], C, full[layer], stream=compute)
        torch.cuda.synchronize()
        gemm = {}
        with torch.cuda.stream(compute):
            for m in tokens + [t for t in iso_tokens if t not in tokens]:
                for _ in range(2):
                    for layer in range(L):
                        b = full[layer].data_ptr()
                        swr.mlp_forward(b + o_gu, scales[layer][0], b + o_d, scales[layer][1], "fp8_e4m3fn", H, I,
                                        xs[m], ys[m], wsp[m], stream=compute)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(compute)
                for _ in range(args.isolated_reps):
                    for layer in range(L):
                        b = full[layer].data_ptr()
                        swr.mlp_forward(b + o_gu, scales[layer][0], b + o_d, scales[layer][1], "fp8_e4m3fn", H, I,
                                        xs[m], ys[m], wsp[m], stream=compute)
                e1.record(compute)
                torch.cuda.synchronize()
                gemm[m] = e0.elapsed_time(e1) / (args.isolated_reps * L)  # ms per layer
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(compute):
            for layer in range(L):
                swr.reassemble_into_slot(chunks[layer], C, full[(layer + 1) % L], stream=compute)
            e0.record(compute)
            for _ in range(args.isolated_reps):
                for layer in range(L):
                    swr.reassemble_into_slot(chunks[layer], C, full[(layer + 1) % L], stream=compute)
            e1.record(compute)
        torch.cuda.synchronize()
        return gemm, e0.elapsed_time(e1) / (args.isolated_reps * L)

    def calibration_copy():
        # a plain device-to-device copy of known size (read + write of the same
        # byte count), the reference that hardware byte counters are scaled by
        if args.calibration_copy_mib > 0:
            src = torch.empty(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(2):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

    if args.isolated_only:
        # only the isolated MLPs (every M) and gathers, then the calibration
        # copy: hardware-counter runs then attribute every GEMM launch to one
        # isolated call at a known token count
        iso_gemm, iso_gather_ms = isolated_kernels()
        calibration_copy()
        print(json.dumps({"isolated_gemm_ms_per_layer": {str(m): round(iso_gemm[m], 4) for m in tokens},
                          "isolated_weight_GBps": {str(m): round((w_bytes + s_bytes) / (iso_gemm[m] * 1e-3) / 1e9, 1)
                                                   for m in tokens},
                          "isolated_reassembly_GBps": round(2 * T / (iso_gather_ms * 1e-3) / 1e9, 1),
                          "isolated_reps": args.isolated_reps}), flush=True)
        planner.close()
        return 0

    # ---------------------------------------------------------------- warmup
    with torch.cuda.stream(compute):
        for _ in range(args.warmup):
            for m in tokens:
                forward(m)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # each forward bracketed by fence-free events, the kind the planner's own
    # timing uses (a default event's system-scope release costs a few us)
    from bench_workloads import FenceFreeEvents

    fwd_ev = FenceFreeEvents(2 * args.steps * len(tokens))
    # The planner times every copy (events on the side stream around it) and
    # every layer's compute (its begin record after the ready wait -- the last
    # packet before the layer's kernels -- to a record after done): no event
    # of the bench sits between a gate and the work it orders.
    sampled = [s for s in range(args.steps) if s % max(1, args.timing_every) == 0]
    planner.set_timing(len(sampled) * len(tokens) * L)
    remote_before, gathers_before = planner.counters()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(compute):
        for s in range(args.steps):
            # in cyclic mode the gather of the next forward's first layer is
            # dispatched during this forward: the sample is the gathers issued
            # in the sampled steps, L per forward as well
            planner.pause_timing(s not in sampled)
            for j, m in enumerate(tokens):
                k = 2 * (s * len(tokens) + j)
                fwd_ev.record(k, compute)
                forward(m)
                fwd_ev.record(k + 1, compute)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    remote_after, gathers_after = planner.counters()
    gathers = planner.gather_times()
    layer_spans = planner.layer_times()
    planner.set_timing(0)
    planner.pause_timing(False)
    assert len(gathers) == len(sampled) * len(tokens) * L and len(layer_spans) == len(gathers)
    # (in cyclic mode the first timed forward's first layer was gathered during warmup, and
    # the last timed forward gathers one layer for a forward that does not run; the count is
    # the same)
    gather_ms = {m: [] for m in tokens}
    k = 0
    for s in sampled:
        for m in tokens:
            gather_ms[m].extend(gathers[k:k + L])
            k += L
    gemm_ms = {m: [] for m in tokens}
    k = 0
    for s in sampled:
        for m in tokens:
            gemm_ms[m].extend(layer_spans[k:k + L])
            k += L
    fwd_ms = {m: [fwd_ev.elapsed_ms(2 * (s * len(tokens) + j), 2 * (s * len(tokens) + j) + 1)
                  for s in range(args.steps)] for j, m in enumerate(tokens)}
    fwd_ev.close()

    ms_per_step = wall * 1e3 / args.steps
    mlp_bytes_per_step = len(tokens) * L * (w_bytes + s_bytes)
    value = mlp_bytes_per_step * args.steps / wall / 1e9

    default_schedule = f"gate_{args.gate}_queues_{args.queues}_lds_{args.gather_lds}"
    iso_gemm, iso_gather_ms = {}, None
    if args.timed_only:
        args.minimal = True  # nothing else after the timed steps
    else:
        iso_gemm, iso_gather_ms = isolated_kernels()

    # The sections below (serial reference, DMA-engine gather, tensor-parallel
    # share, graph replay) are reports beside the headline; --minimal skips
    # them, e.g. for hardware-counter runs that average over every MLP call.
    serial_ms, serial_bare_ms, dma, graph, tpres, schedules, R, rank_bytes = {}, {}, {}, {}, {}, {}, 4, 0
    pipelined_bare_ms, bare_trials, serial_timed_ms = {}, {}, {}
    if not args.minimal:
        # ---------------------------------------------------------------- serial reference
        # the same gathers and MLPs back to back on one stream, without the
        # planner, at three levels of instrumentation: "timed" (fence-free
        # events around each gather, each MLP and the forward, as in the timed
        # steps the planner times), "bracketed" (the forward's two events only,
        # as in the other timed steps) and bare (no events, timed in trials
        # that alternate with the default schedule's bare forwards, median of
        # each, so that both see the same clocks and temperature).
        from bench_workloads import FenceFreeEvents

        fwd_reps = max(4, args.steps // 2)

        def time_forwards(pl, m, reps=fwd_reps):
            with torch.cuda.stream(compute):
                forward(m, pl=pl)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(compute)
                for _ in range(reps):
                    forward(m, pl=pl)
                e1.record(compute)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ev_pool = FenceFreeEvents(4 * L + 2)

        def serial_forward(m, level):
            # level 0: bare, 1: the forward bracketed, 2: every gather and MLP timed too
            if level:
                ev_pool.record(4 * L, compute)
            for layer in range(L):
                s_ = slot_a if layer % 2 == 0 else slot_b
                if level > 1:
                    ev_pool.record(4 * layer, compute)
                swr.reassemble_into_slot(chunks[layer], C, s_, stream=compute)
                if level > 1:
                    ev_pool.record(4 * layer + 1, compute)
                    ev_pool.record(4 * layer + 2, compute)
                b = s_.data_ptr()
                swr.mlp_forward(b + o_gu, scales[layer][0], b + o_d, scales[layer][1], "fp8_e4m3fn", H, I,
                                xs[m], ys[m], wsp[m], stream=compute)
                if level > 1:
                    ev_pool.record(4 * layer + 3, compute)
            if level:
                ev_pool.record(4 * L + 1, compute)

        def time_serial(m, level, reps=fwd_reps):
            with torch.cuda.stream(compute):
                serial_forward(m, level)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(compute)
                for _ in range(reps):
                    serial_forward(m, level)
                e1.record(compute)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        for m in tokens:
            serial_timed_ms[m] = time_serial(m, 2)
            serial_ms[m] = time_serial(m, 1)
            ts, tp = [], []
            for _ in range(3):
                ts.append(time_serial(m, 0))
                tp.append(time_forwards(planner, m))
            serial_bare_ms[m], pipelined_bare_ms[m] = float(np.median(ts)), float(np.median(tp))
            bare_trials[m] = {"serial": [round(t, 4) for t in ts], "pipelined": [round(t, 4) for t in tp]}
        ev_pool.close()

        # ---------------------------------------------------------------- schedules
        # The same forwards under every gate, on two streams and on one queue,
        # without timing events (ms per 8-layer forward).  On one GPU the
        # gather (2|T| bytes) and the MLP (|T| bytes) draw on one HBM.
        combos = [("done", 2, 0), ("begin", 2, 0), ("after", 2, 0), ("done", 2, YIELD_LDS), ("begin", 2, YIELD_LDS),
                  ("done", 1, 0), ("after", 1, 0)]
        if (args.gate, args.queues, args.gather_lds) not in combos:
            combos.append((args.gate, args.queues, args.gather_lds))
        for gname, q, lds in combos:
            pl = make_planner(gname, q, lds)
            schedules[f"gate_{gname}_queues_{q}_lds_{lds}"] = {str(m): round(time_forwards(pl, m), 4) for m in tokens}
            pl.close()

        # ---------------------------------------------------------------- DMA-engine gather
        # the pages' gate with the gathers on the DMA engines (no compute
        # units): the copy-engine path, at the smallest and largest M
        dma = {}
        dpl = make_planner("done", 2)
        dpl.set_copy_engine(swr.ENGINE_DMA)
        dma_steps = max(2, args.steps // 4)
        for m in sorted({tokens[0], tokens[-1]}):
            with torch.cuda.stream(compute):
                forward(m, pl=dpl)
            torch.cuda.synchronize()
            evd = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
                   for _ in range(dma_steps)]
            fwd_d = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(dma_steps)]
            with torch.cuda.stream(compute):
                for s in range(dma_steps):
                    fwd_d[s][0].record(compute)
                    forward(m, evd[s], pl=dpl)
                    fwd_d[s][1].record(compute)
            torch.cuda.synchronize()
            f = float(np.median([a.elapsed_time(b) for a, b in fwd_d]))
            g = float(np.mean([a.elapsed_time(b) for row in evd for a, b in row]))
            dma[str(m)] = {"pipelined_ms_per_forward": round(f, 4), "gemm_ms_per_layer_in_pipeline": round(g, 4),
                           "gemm_slowdown_vs_isolated": round(g / iso_gemm[m], 3)}
        dpl.close()

        # ---------------------------------------------------------------- tensor-parallel share
        # The PR report's alternative to weight sharding: each of R ranks (its
        # deployment's TP4) holds 1/R of the intermediate dimension and computes an
        # fp32 partial of Y; the partials are all-reduced.  One GPU shows one
        # rank's share at its real shape, timed over all ranks' shards of all
        # layers (so no cache serves a later call), and the local reduce of R
        # partials.
        R = 4
        sh = I // R
        tmp = torch.empty(T, dtype=torch.uint8, device=dev)
        shards = []
        for layer in range(L):
            swr.reassemble_into_slot(chunks[layer], C, tmp, stream=compute)
            torch.cuda.synchronize()
            gu_full = tmp[o_gu:o_gu + 2 * I * H].view(2 * I, H)
            d_full = tmp[o_d:o_d + H * I].view(H, I)
            for r in range(R):
                rows = torch.cat([torch.arange(r * sh, (r + 1) * sh), torch.arange(I + r * sh, I + (r + 1) * sh)]).to(dev)
                shards.append((gu_full.index_select(0, rows).contiguous(), scales[layer][0].index_select(0, rows).contiguous(),
                               d_full[:, r * sh:(r + 1) * sh].contiguous(), scales[layer][1]))
            torch.cuda.synchronize()
        del tmp
        rank_bytes = 2 * sh * H + H * sh + (2 * sh + H) * 4
        tpres = {}
        for m in sorted({tokens[0], tokens[-1]}):
            parts = [torch.empty((m, H), dtype=torch.float32, device=dev) for _ in range(R)]
            yt = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
            wst = torch.empty(swr.mlp_workspace_bytes(m, H, sh, "fp8_e4m3fn"), dtype=torch.uint8, device=dev)

            def rank_pass(m=m, parts=parts, wst=wst):
                for i, (g_r, sg_r, d_r, sd_r) in enumerate(shards):
                    swr.mlp_forward_partial(g_r, sg_r, d_r, sd_r, "fp8_e4m3fn", H, sh, xs[m], parts[i % R], wst,
                                            stream=compute)

            with torch.cuda.stream(compute):
                rank_pass()
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(compute)
                rank_pass()
                e1.record(compute)
                for _ in range(L):
                    swr.sum_partials(parts, yt, stream=compute)
                e2.record(compute)
            torch.cuda.synchronize()
            rank_ms = e0.elapsed_time(e1) / len(shards)
            red_ms = e1.elapsed_time(e2) / L
            tpres[str(m)] = {"rank_mlp_ms_per_layer": round(rank_ms, 4),
                             "rank_weight_GBps": round(rank_bytes / (rank_ms * 1e-3) / 1e9, 1),
                             "reduce_of_partials_ms": round(red_ms, 4),
                             "weight_sharded_serial_ms_per_layer": round(serial_ms[m] / L, 4)}
        del shards

        # ---------------------------------------------------------------- graph replay
        # one forward captured as a graph (weight_sharding, CUDA graph section)
        # and replayed, against the same planner run eagerly:
        #   * without a prefetch: the captured forward gathers its first layer
        #     itself, so every replay stands alone;
        #   * with the first layer gathered on a dedicated stream outside the
        #     graph (swr_planner_set_first_prefetch): each replay's prefetch for
        #     the next replay is enqueued right behind it and overlaps its last
        #     layer; the graph waits for it.
        graph = {}
        reps = max(4, args.steps // 2)
        pf_stream = torch.cuda.Stream()
        for mode in ("no_prefetch", "first_layer_prefetch_stream"):
            gp = swr.Planner(0, L, compute, side, slot_a, slot_b)
            gp.set_gate(gate_of[args.gate])
            for layer in range(L):
                gp.set_layer(layer, chunks[layer], C)
            pre = mode != "no_prefetch"
            if pre:
                gp.set_first_prefetch(pf_stream)
                gp.prefetch_first()
            row = {}
            for m in sorted({tokens[0], tokens[-1]}):
                def eager_fwd():
                    forward(m, pl=gp)
                    if pre:
                        gp.prefetch_first()
                with torch.cuda.stream(compute):
                    eager_fwd()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(compute):
                    e0.record(compute)
                    for _ in range(reps):
                        eager_fwd()
                    e1.record(compute)
                torch.cuda.synchronize()
                eager = e0.elapsed_time(e1) / reps
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=compute):
                    forward(m, pl=gp)
                g.replay()
                if pre:
                    gp.prefetch_first()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(compute):
                    e0.record(compute)
                    for _ in range(reps):
                        g.replay()
                        if pre:
                            gp.prefetch_first()
                    e1.record(compute)
                torch.cuda.synchronize()
                row[str(m)] = {"eager_ms_per_forward": round(eager, 4),
                               "graph_replay_ms_per_forward": round(e0.elapsed_time(e1) / reps, 4)}
                del g
            graph[mode] = row
            gp.close()

    # ---------------------------------------------------------------- roofline
    def mlp_alg_bytes(m: int) -> int:
        # weights + scales + X read + h write + h read + Y write
        return w_bytes + s_bytes + m * H * 2 + 2 * m * I * 2 + m * H * 2

    gemm_avg = {m: float(np.mean(gemm_ms[m])) for m in tokens}
    gather_avg = float(np.mean([v for m in tokens for v in gather_ms[m]]))
    per_kernel = {
        "mlp_forward": {
            "kernels": "staged_gemm_kernel (gate_up with SiLU*up) + staged_gemm_kernel (down) "
                       "[+ splitk_finalize_kernel]",
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "bytes_per_launch": {str(m): mlp_alg_bytes(m) for m in tokens},
            "avg_ms": {str(m): gemm_avg[m] for m in tokens},
            "achieved": sum(mlp_alg_bytes(m) for m in tokens) / (sum(gemm_avg[m] for m in tokens) * 1e-3) / 1e9,
            "frac_by_tokens": {str(m): round(mlp_alg_bytes(m) / (gemm_avg[m] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                               for m in tokens},
        },
        "reassemble_into_slot": {
            "kernels": "reassemble_kernel",
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS, "bytes_per_launch": 2 * T,
            "avg_ms": gather_avg, "achieved": 2 * T / (gather_avg * 1e-3) / 1e9,
        },
    }
    for k in per_kernel.values():
        k["frac"] = k["achieved"] / k["peak"]
        k["traffic"] = None
    for name, k in per_kernel.items():
        k["traffic"] = measured_traffic(name)
    # The roofline names the decode MLP, the metric's own kernels: each call's
    # duration is the span the planner records on the compute stream from the
    # layer's begin (after its ready wait) to just after its done record, which
    # holds the MLP's launches and nothing else; bytes are the algorithmic
    # bytes of one call.  The gather's kernel is reported beside it.
    dk = per_kernel["mlp_forward"]
    tr = dk["traffic"]
    if isinstance(tr, dict):  # per token count -> per launch, averaged over the token counts
        tr = int(sum(tr[str(m)] for m in tokens) / len(tokens)) if all(str(m) in tr for m in tokens) else None
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 1), "peak": dk["peak"], "unit": dk["unit"],
                "frac": round(dk["frac"], 4), "traffic": tr, "kernel": "mlp_forward",
                "kernels": dk["kernels"], "target_frac": 0.80,
                "target_met": bool(min(dk["frac_by_tokens"].values()) >= 0.80)}

    per_m = {}
    for m in tokens:
        # forwards without the planner's timing records (the forward's own two
        # events only), and the sampled ones that carry them; means, like the
        # serial references'
        plain = [t for s, t in enumerate(fwd_ms[m]) if s not in sampled]
        fwd = float(np.mean(plain if plain else fwd_ms[m]))
        fwd_timed = float(np.mean([fwd_ms[m][s] for s in sampled]))
        g_layer = float(np.mean(gather_ms[m]))
        per_m[str(m)] = {
            "pipelined_ms_per_forward": round(fwd, 4),
            "pipelined_tokens_per_s": round(m / (fwd * 1e-3), 1),
            "pipelined_weight_GBps": round(L * (w_bytes + s_bytes) / (fwd * 1e-3) / 1e9, 1),
            "pipelined_hbm_frac": round(L * (3 * T + mlp_alg_bytes(m) - w_bytes) / (fwd * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "compute_stall_ms": round(fwd - L * gemm_avg[m], 4),
            "gemm_ms_per_layer_in_pipeline": round(gemm_avg[m], 4),
            "gather_ms_per_layer_in_pipeline": round(g_layer, 4),
            # the pages' evaluation: per layer, gather time over compute time,
            # and the part of a layer's wall time that is not its GEMMs
            "gather_to_compute_ratio": round(g_layer / gemm_avg[m], 3),
            "exposed_ms_per_layer": round(fwd / L - gemm_avg[m], 4),
            **({} if m not in iso_gemm else {
                "isolated_gemm_ms_per_layer": round(iso_gemm[m], 4),
                "isolated_weight_GBps": round((w_bytes + s_bytes) / (iso_gemm[m] * 1e-3) / 1e9, 1),
                "isolated_weight_frac": round((w_bytes + s_bytes) / (iso_gemm[m] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "isolated_tokens_per_s": round(m / (L * iso_gemm[m] * 1e-3), 1),
                "isolated_gather_to_compute_ratio": round(iso_gather_ms / iso_gemm[m], 3)}),
            "serial_reference_ms_per_forward": round(serial_ms[m], 4) if m in serial_ms else None,
            "pipelined_timed_ms_per_forward": round(fwd_timed, 4),
            "serial_reference_timed_ms_per_forward": round(serial_timed_ms[m], 4) if m in serial_timed_ms else None,
            "serial_reference_bare_ms_per_forward": round(serial_bare_ms[m], 4) if m in serial_bare_ms else None,
            "pipelined_bare_ms_per_forward": round(pipelined_bare_ms[m], 4) if m in pipelined_bare_ms else None,
            "bare_trials_ms_per_forward": bare_trials.get(m),
        }

    # ---------------------------------------------------------------- accounts
    # weight_sharding, cost section: received bytes per layer (N-1)/N * |T| and
    # per-rank weight memory R/N + 2 max|T_l|, from the library's own layouts
    # and the planner's transfer counter over the timed steps
    lays = [swr.plan_layer(shp, N)[1] for _ in range(L)]
    r_total = sum(l_["total_bytes"] for l_ in lays)
    per_rank = sum(l_["chunk_bytes"] for l_ in lays)
    timed_gathers = gathers_after - gathers_before
    accounts = {
        "transfer_bytes_counted": remote_after - remote_before,
        "gathers_counted": timed_gathers,
        "transfer_bytes_per_gather": (remote_after - remote_before) // max(1, timed_gathers),
        "transfer_bytes_per_gather_expected": (N - 1) * C,
        "replicated_weight_bytes_R": r_total,
        "resident_chunk_bytes_per_rank_R_over_N": per_rank,
        "slot_bytes_2_max_T": 2 * max(l_["total_bytes"] for l_ in lays),
        "weight_memory_per_rank": per_rank + 2 * max(l_["total_bytes"] for l_ in lays),
        "all_chunks_on_this_gpu": N * per_rank,
    }

    calibration_copy()

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, H, I, x_all, tokens)

    result = {
        "metric": "decode MLP weight-stream GB/s + tokens/s at M=1..64 (fraction of HBM peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn weights x bf16 activations, fp32 accumulate",
        "data": "synthetic: seeded N(0,0.02) weights quantised per row to E4M3FN, N(0,1) bf16 tokens",
        "config": {
            "workload": wl.name, "hidden": H, "intermediate": I, "layers": L, "n_chunks": N,
            "tokens": tokens, "layer_bytes": T, "chunk_bytes": C, "slots": 2, "gate": args.gate,
            "queues": args.queues, "gather_lds": args.gather_lds,
            "step": "pipelined forward (reassembly + MLP per layer through the planner) over all layers for every M",
        },
        "value_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "per_tokens": per_m,
        # the isolated MLP at every token count timed, headline and curve alike
        "isolated_curve": {str(m): {"ms_per_layer": round(g, 4),
                                    "weight_GBps": round((w_bytes + s_bytes) / (g * 1e-3) / 1e9, 1),
                                    "weight_frac": round((w_bytes + s_bytes) / (g * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
                           for m, g in sorted(iso_gemm.items())},
        "isolated_reassembly_GBps": round(2 * T / (iso_gather_ms * 1e-3) / 1e9, 1) if iso_gather_ms else None,
        "schedules_ms_per_forward": schedules,
        "dma_engine_gather": dma,
        "graph_replay": graph,
        "tensor_parallel_share": {"ranks": R, "rank_weight_bytes_per_layer": rank_bytes, "per_tokens": tpres},
        "accounts": accounts,
        "roofline": roofline,
        "roofline_by_kernel": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                               for k, v in per_kernel.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    planner.close()
    return 0


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 --pmc summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the counter's reading for a plain
    copy of known size), or None if there is none or the kernel's sources changed
    since the counters were taken.  For mlp_forward, a dict by token count."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic_shared_expert_decode.json")
    try:
        rec = json.load(open(path))[kernel]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != rec["source_sha"]:
            return None
        b = rec["bytes_per_launch"]
        return {k: int(v) for k, v in b.items()} if isinstance(b, dict) else int(b)
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, H, I, x_all, tokens) -> dict:
    """The oracle (float64 NumPy, untuned) on one layer at the largest M."""
    import numpy as np

    import synth
    from oracle import gemm

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    gu, d = wl.layer_weights(0)
    m = max(tokens)
    times = []
    for _ in range(2):
        t = time.perf_counter()
        gemm.mlp(x_all[:m], gu.raw(), gu.scale, d.raw(), d.scale, gu.dtype, H, I)
        times.append(time.perf_counter() - t)
    best = min(times)
    wb = gu.nbytes + d.nbytes + (2 * I + H) * 4
    log(f"cpu oracle one layer at M={m}: {best:.2f}s")
    return {
        "value": round(wb / best / 1e9, 3),
        "unit": "GB/s",
        "tokens_per_s": round(m / (best * wl.layers), 3),
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"one shared-expert layer (of {wl.layers}) at M={m}, float64 NumPy oracle, best of 2 runs; "
                  f"tokens/s scaled to the {wl.layers}-layer stack",
    }


if __name__ == "__main__":
    sys.exit(main())
