"""The library's calls recorded into a HIP graph (torch.cuda.CUDAGraph, which is
a HIP graph on ROCm) and replayed: every kernel reads its arguments from the
launch, none allocates or sets memory, so each replay must equal the same call
made eagerly, bit for bit.  Each graph is replayed several times, with eager
work and synchronisations between the replays, and every replay is checked."""
import pytest
import torch

import workloads
from kda_testutil import dev, gpu_or_skip

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def capture(fn):
    """Warm up on a side stream (as torch requires), then record fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_decode_step_graph_replays():
    """A decode step advancing states in place: three replays equal three eager
    steps from the same starting states."""
    m = kda()
    inp = workloads.decode_batch(B=32)
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    s0 = dev(inp.S0)
    s_eager = s0.clone()
    outs = [m.kda_decode_step(q, k, v, g, b, s_eager).clone() for _ in range(3)]
    states = []
    s_eager2 = s0.clone()
    for _ in range(3):
        m.kda_decode_step(q, k, v, g, b, s_eager2)
        states.append(s_eager2.clone())
    s_graph = s0.clone()
    o_graph = torch.empty_like(outs[0])
    graph = capture(lambda: m.kda_decode_step(q, k, v, g, b, s_graph, o=o_graph))
    s_graph.copy_(s0)  # the warm-up call advanced it once
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, outs[r]), r
        assert torch.equal(s_graph, states[r]), r
        _ = (q.float() * 2).sum().item()  # eager work between replays


def test_prefill_graph_replays():
    """The two-kernel prefill (window plan fixed at capture) and a state init in
    one graph: three replays equal the eager call."""
    m = kda()
    inp = workloads.recurrence_inputs([200, 70, 1], H=4, d=128, dtype="bf16", chunk=64,
                                      s0_std=0.05, seed=77)
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu, cuh = dev(inp.cu_seqlens), inp.cu_seqlens
    s0 = dev(inp.S0)
    need = m.kda_prefill_workspace_bytes_batch(cuh, 4, 128, 128, 64, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_e, S_e = m.kda_prefill_chunked(q, k, v, g, b, cu_seqlens=cu, cu_seqlens_host=cuh,
                                     initial_state=s0, workspace=ws)
    torch.cuda.synchronize()
    o_e, S_e = o_e.clone(), S_e.clone()
    state = torch.empty_like(s0)
    o = torch.empty_like(o_e)
    S = torch.empty_like(S_e)

    def call():
        m.kda_state_init(state, s0)
        m.kda_prefill_chunked(q, k, v, g, b, cu_seqlens=cu, cu_seqlens_host=cuh,
                              initial_state=state, final_state=S, o=o, workspace=ws)

    graph = capture(call)
    for r in range(3):
        o.zero_()
        S.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), r
        assert torch.equal(S, S_e), r
