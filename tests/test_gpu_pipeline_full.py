"""The lookahead / ping-pong pipeline at full size (weight_sharding,
zdszero.github.io, section "lookahead and ping-pong slot").

Four distinct shared-expert layers (hidden 6144, intermediate 14336, FP8,
264,241,152 bytes each, N = 16 chunks of 16,515,072 bytes) run through the
planner at 1 and 64 tokens, two forwards back to back, in cyclic mode.  The
gather of layer l+1 then really races the 40-150 us GEMMs of layer l that
read the other slot, and the next forward's first gather races the last
layer.  For every forward and layer:
  * all of h (the gate_up -> SiLU*up output, read from that layer's own
    workspace) and sampled columns of Y are checked against the oracle;
  * the planner's trace equals the oracle's model and passes its
    happens-before checker;
  * the counted transfer bytes are 15 C per gather.
A gather that overwrote a slot still being read, or a layer that read the
other slot, would put another layer's weights into some layer's output.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import gemm, numerics
from oracle import scheduler as osch

from gpu_util import DEV, assert_close_rows, bf16, f32, note, u8

pytestmark = pytest.mark.gpu

N_LAYERS = 4
M_MAX = 64
N_COLS = 384


@pytest.fixture(scope="module")
def stack():
    wl = synth.SHARED_EXPERT_DECODE
    H, I, N = wl.hidden, wl.intermediate, wl.n_chunks
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, N)
    assert lay["total_bytes"] == 264_241_152 and lay["chunk_bytes"] == 16_515_072
    x = synth.activations(synth.seed_for(2, 0, 50), M_MAX, H)
    cols = np.sort(np.random.default_rng(7).choice(H, size=N_COLS, replace=False))
    layers = []
    for layer in range(N_LAYERS):
        note(f"pipeline stack: generating and packing layer {layer}")
        gu, d = wl.layer_weights(layer)
        chunks = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(N)]
        swr.pack_layer(lay, views, [u8(gu.raw()), u8(d.raw())], chunks)
        torch.cuda.synchronize()
        g = gemm.proj_f64(x, gu.raw(), gu.dtype, 2 * I, H, gu.scale)
        with np.errstate(over="ignore"):
            h = numerics.f64_to_bf16_bits(numerics.silu(g[:, :I]) * g[:, I:])
        del g
        y = gemm.proj_f64(h, np.ascontiguousarray(d.data[cols]), d.dtype, len(cols), I, d.scale[cols])
        layers.append(dict(chunks=chunks, s_gu=f32(gu.scale), s_d=f32(d.scale), h_ref=h, y_ref=y))
    slot_a = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=DEV)
    return dict(wl=wl, views=views, lay=lay, x=x, xd=bf16(x), cols=cols, layers=layers, slots=(slot_a, slot_b))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("m", [1, 64])
@pytest.mark.parametrize("gate,gather_lds,one_queue", [(swr.GATE_DONE, 0, False), (swr.GATE_BEGIN, 57344, False),
                                                       (swr.GATE_DONE, 57344, False), (swr.GATE_AFTER, 0, False),
                                                       (swr.GATE_AFTER, 0, True)])
def test_full_size_pipeline_matches_oracle(stack, m, gate, gather_lds, one_queue):
    wl, lay, views = stack["wl"], stack["lay"], stack["views"]
    H, I, C = wl.hidden, wl.intermediate, lay["chunk_bytes"]
    note(f"full-size pipeline m={m} gate={gate} gather_lds={gather_lds} one_queue={one_queue}")
    compute = torch.cuda.Stream()
    side = compute if one_queue else torch.cuda.Stream()
    slot_a, slot_b = stack["slots"]
    # garbage in both slots: a layer that computed before its gather landed would show it
    slot_a.fill_(0x7F)
    slot_b.fill_(0x7F)
    torch.cuda.synchronize()
    p = swr.Planner(0, N_LAYERS, compute, side, slot_a, slot_b)
    for i, L in enumerate(stack["layers"]):
        p.set_layer(i, L["chunks"], C)
    p.set_cyclic(True)
    p.set_gate(gate)
    p.set_gather_lds(gather_lds)
    o_gu, o_d = views[0]["offset"], views[1]["offset"]
    xd = stack["xd"][:m]
    n_fwd = 2
    ys = [[torch.full((m, H), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(N_LAYERS)]
          for _ in range(n_fwd)]
    wsb = swr.mlp_workspace_bytes(m, H, I, "fp8_e4m3fn")
    wss = [[torch.empty(wsb, dtype=torch.uint8, device=DEV) for _ in range(N_LAYERS)] for _ in range(n_fwd)]
    traces = []
    with torch.cuda.stream(compute):
        for f in range(n_fwd):
            p.reset()
            p.pre_dispatch(0)
            for layer in range(N_LAYERS):
                p.maybe_dispatch(layer + 1)
                base = p.wait_ready_once(layer)
                L = stack["layers"][layer]
                swr.mlp_forward(base + o_gu, L["s_gu"], base + o_d, L["s_d"], "fp8_e4m3fn", H, I, xd, ys[f][layer],
                                wss[f][layer], stream=compute)
                p.update_done_event(layer)
            traces.append(p.trace())
    torch.cuda.synchronize()
    g = {swr.GATE_DONE: "done", swr.GATE_BEGIN: "begin", swr.GATE_AFTER: "after"}[gate]
    assert traces[0] == osch.expected_trace(0, N_LAYERS, prefetched=False, prefetch_next=True, gate=g)
    assert traces[1] == osch.expected_trace(0, N_LAYERS, prefetched=True, prefetch_next=True, gate=g)
    assert osch.check_trace(traces) == []
    remote, gathers = p.counters()
    assert gathers == n_fwd * N_LAYERS + 1
    assert remote == gathers * 15 * 16_515_072
    cols = stack["cols"]
    for f in range(n_fwd):
        for layer in range(N_LAYERS):
            L = stack["layers"][layer]
            h = wss[f][layer][:m * I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(m, I)
            assert_close_rows(numerics.bf16_to_f64(h), numerics.bf16_to_f64(L["h_ref"][:m]),
                              what=f"forward {f} layer {layer} h")
            y = ys[f][layer].float().cpu().numpy().astype(np.float64)
            assert_close_rows(y[:, cols], L["y_ref"][:m], what=f"forward {f} layer {layer} y")
    p.set_cyclic(False)
    p.close()
