"""The C-ABI calls under HIP graph capture: decode steps, a prefill and the
one-call layer recurrence, with every buffer (outputs, state, workspace)
allocated before capture, are recorded into a torch.cuda.CUDAGraph and
replayed several times, with eager work and synchronizations between
replays; every replay must equal the eager result bit for bit. (The kernels allocate nothing and issue no memset,
so a captured call is exactly its launches.)"""
import pytest
import torch

import gated_delta_rule_72_amd as kda
from gated_delta_rule_72_amd import workloads as wl

from gpu_util import custom, device

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_equal_eager_steps():
    dev = device()
    w = custom("graph_decode", H=4, d=128, lens=(1,) * 32, gate="per_key", s0_std=0.05, seed=90)
    inp = wl.make_decode_inputs(w, dev)
    shape = kda.make_shape(w.H, w.dk, w.dv, inp["q"].dtype, True)
    B = w.num_seqs
    state_eager = inp["state"].clone()
    state_graph = inp["state"].clone()
    o_eager = torch.empty((B, w.H, w.dv), dtype=torch.float32, device=dev)
    o_graph = torch.empty_like(o_eager)
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up outside capture
        kda.kda_decode_step(shape, B, *args, state_graph.clone(), torch.empty_like(o_graph))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.kda_decode_step(shape, B, *args, state_graph, o_graph)
    # capture recorded the launch without running it: state_graph is unchanged
    torch.cuda.synchronize()
    assert torch.equal(state_graph, inp["state"])
    for rep in range(4):
        kda.kda_decode_step(shape, B, *args, state_eager, o_eager)
        torch.cuda.synchronize()
        junk = torch.randn(1024, device=dev).sum()          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), rep
        assert torch.equal(state_graph, state_eager), rep
        del junk


def test_prefill_graph_replays_equal_eager_call():
    dev = device()
    w = custom("graph_prefill", H=2, d=64, lens=(300, 65, 0, 7), gate="scalar", s0_std=0.02, interval=64, seed=91)
    inp = wl.make_prefill_inputs(w, dev)
    shape = kda.make_shape(w.H, w.dk, w.dv, inp["q"].dtype, False)
    cu_h = inp["cu_seqlens_host"]
    n_snap = kda.kda_snapshot_count(cu_h, w.interval)
    f32 = dict(dtype=torch.float32, device=dev)

    def buffers():
        return (torch.empty((w.T, w.H, w.dv), **f32), torch.empty((w.num_seqs, w.H, w.dv, w.dk), **f32),
                torch.empty((n_snap, w.H, w.dv, w.dk), **f32))

    ws = torch.empty(kda.kda_prefill_workspace_size(shape, cu_h, 64, w.interval), dtype=torch.uint8, device=dev)

    def call(o, fin, snaps):
        kda.kda_prefill_chunked(shape, cu_h, inp["cu_seqlens"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                                inp["beta"], inp["initial_state"], o, fin, snaps, ws,
                                snapshot_interval=w.interval)

    eager = buffers()
    call(*eager)
    torch.cuda.synchronize()
    graph_out = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(*graph_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for t in graph_out:
        t.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(*graph_out)
    for rep in range(3):
        for t in graph_out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(graph_out, eager):
            assert torch.equal(x, y), rep


@pytest.mark.parametrize("gate,d", [("scalar", 128), ("per_key", 64)])
def test_layer_prefill_graph_replays_equal_eager_call(gate, d):
    """kda_layer_prefill in its fused form (every sequence split into 256-token
    segments) under capture: each replay equals the eager call bit for bit."""
    dev = device()
    w = custom(f"graph_layer_{gate}", H=2, d=d, lens=(700, 300), gate=gate, s0_std=0.02, seed=92)
    inp = wl.make_prefill_inputs(w, dev)
    li = wl.make_layer_inputs(w, dev, seed=93)
    g_logit = li["g_logit"].to(torch.bfloat16)
    shape = kda.make_shape(w.H, w.dk, w.dv, inp["q"].dtype, gate == "per_key")
    cu_h = inp["cu_seqlens_host"]
    ws = torch.empty(kda.kda_layer_prefill_workspace_size(shape, cu_h, 64, 0, 256), dtype=torch.uint8, device=dev)

    def buffers():
        return (torch.empty((w.T, w.H, w.dv), dtype=torch.bfloat16, device=dev),
                torch.empty((w.num_seqs, w.H, w.dv, w.dk), dtype=torch.float32, device=dev))

    def call(out, fin):
        kda.kda_layer_prefill(shape, cu_h, inp["cu_seqlens"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                              inp["beta"], inp["initial_state"], g_logit, li["norm_w"], 1e-6, kda.KDA_BF16, out,
                              fin, None, ws, segment_tokens=256)

    eager = buffers()
    call(*eager)
    torch.cuda.synchronize()
    graph_out = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(*graph_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(*graph_out)
    for rep in range(3):
        for t in graph_out:
            t.fill_(float("nan"))
        junk = torch.randn(1024, device=dev).sum()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(graph_out, eager):
            assert torch.equal(x, y), rep
        del junk
