"""The decode and prefill steps allocate nothing and the library issues no memsets, so a step
captured in a HIP graph (torch.cuda.CUDAGraph) must replay exactly: every replay is compared with
an eager run on the same inputs, with unrelated eager work and input changes between replays."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from top_fp4_lightning_amd import pipeline

    return pipeline


def snapshot(plan):
    return [t.clone() for t in plan.topk + plan.topk_val + [plan.pool_blocks, plan.pool_count, plan.block_max]]


def assert_same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), what


def test_decode_step_graph_replays_match_eager(pl):
    wl = synth.decode_workload("g", 91, [40000, 70001, 9000], layers=2)
    dev = pl.DeviceWorkload.from_workload(wl)
    plan = pl.DecodePlan(dev)
    other = pl.DecodePlan(pl.DeviceWorkload.from_workload(synth.decode_workload("h", 92, [30000], layers=1)))
    plan.run()
    torch.cuda.synchronize()
    eager = snapshot(plan)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        plan.run(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(stream=torch.cuda.current_stream())
    for rep in range(3):
        other.run()  # unrelated eager work between replays
        torch.cuda.synchronize()
        for t in plan.topk + plan.topk_val:  # stale outputs would show
            t.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(plan), eager, f"replay {rep}")

    # new inputs in the captured buffers: the replay must follow them like an eager step
    g = torch.Generator(device="cpu").manual_seed(5)
    for layer in range(len(dev.w)):
        dev.w[layer].copy_(torch.randn(dev.w[layer].shape, generator=g) / 6.0)
    graph.replay()
    torch.cuda.synchronize()
    replayed = snapshot(plan)
    plan.run()
    torch.cuda.synchronize()
    assert_same(replayed, snapshot(plan), "replay after an input change")


def test_prefill_step_graph_replays_match_eager(pl):
    wl = synth.prefill_workload("gp", 93, 20000, 64)
    dev = pl.DeviceWorkload.from_workload(wl)
    plan = pl.PrefillPlan(dev).run()
    torch.cuda.synchronize()
    eager = plan.topk.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(stream=torch.cuda.current_stream())
    for rep in range(3):
        plan.topk.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.topk, eager), f"replay {rep}"
