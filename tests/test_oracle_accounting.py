"""Pins for the memory and transfer accounting (weight-sharding page, cost
section: per-rank transfer about (N-1)/N * S, memory R/N + 2 * max_l |T_l|)."""
import json
import os

from oracle import accounting, layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_shared_expert_stack():
    # 8 layers of 264,241,152 B at N=16: R = 2,113,929,216; R/N = 132,120,576;
    # slots 2 * 264,241,152 = 528,482,304; sum 660,602,880.
    t = [264241152] * 8
    assert accounting.replicated_memory(t) == 2113929216
    assert accounting.resident_per_rank(t, 16) == 132120576
    assert accounting.slot_bytes(t) == 528482304
    assert accounting.weight_shard_memory(t, 16) == 660602880
    # per layer: 15 chunks of 16,515,072 B arrive = 247,726,080 = 15/16 * |T|
    assert accounting.transfer_bytes(264241152, 16) == 247726080
    assert accounting.transfer_bytes(264241152, 16) * 16 == 15 * 264241152


def test_slots_follow_largest_layer():
    small = layout.plan_layer([(8, 8, "bf16")], 4)["total"]
    big = layout.plan_layer([(64, 64, "bf16")], 4)["total"]
    assert accounting.slot_bytes([small, big, small]) == 2 * big
    assert accounting.weight_shard_memory([small, big], 4) == (small + big) // 4 + 2 * big


def test_transfer_matches_layout_remote_bytes():
    for n in (1, 2, 3, 8, 16):
        p = layout.plan_layer([(100, 127, "bf16"), (3, 5, "fp8_e4m3fn")], n)
        assert accounting.transfer_bytes(p["total"], n) == layout.remote_bytes(p)
    assert accounting.transfer_bytes(layout.plan_layer([(4, 4, "bf16")], 1)["total"], 1) == 0


def test_pages_memory_figures_are_consistent():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    rep = fig["replicated_per_card"]
    assert round(sum(rep["parts_GiB"]), 1) == rep["total_GiB"]
    moe = fig["moe_peripheral_reclaimed"]
    assert round(moe["layer_MB"] * 1e6 * moe["layers"] / 2 ** 30, 2) == moe["reclaimed_GiB"]
