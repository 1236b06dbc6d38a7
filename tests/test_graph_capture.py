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


def test_decode_tokens_graph_replays():
    """Multi-token decode (3 tokens per sequence, per-token snapshots, bf16
    states through a slot table) recorded once: every replay equals the eager
    call from the same starting states, outputs and snapshots included."""
    m = kda()
    B, n_tok, H, d, n_slots = 8, 3, 4, 128, 12
    inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype="bf16", s0_std=0.3, seed=81)
    t = lambda x: dev(x.reshape((B, n_tok) + tuple(x.shape[1:])))
    q, k, v, g, b = (t(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    slots = dev(torch.tensor([11, 0, 5, 3, 9, 1, 7, 2], dtype=torch.int32))
    pool = torch.zeros((n_slots, H, d, d), dtype=torch.bfloat16, device="cuda")
    pool[slots.long()] = dev(inp.S0).to(torch.bfloat16)
    want = []
    s_eager = pool.clone()
    for _ in range(3):
        o, snaps = m.kda_decode_tokens(q, k, v, g, b, s_eager, slot_idx=slots, token_states=True)
        want.append((o.clone(), snaps.clone(), s_eager.clone()))
    s_graph = pool.clone()
    o_graph = torch.empty_like(want[0][0])
    snap_graph = torch.empty_like(want[0][1])
    graph = capture(lambda: m.kda_decode_tokens(q, k, v, g, b, s_graph, slot_idx=slots,
                                                o=o_graph, token_states=snap_graph))
    s_graph.copy_(pool)  # the warm-up call advanced it once
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, want[r][0]), r
        assert torch.equal(snap_graph, want[r][1]), r
        assert torch.equal(s_graph, want[r][2]), r
        _ = (v.float() * 2).sum().item()  # eager work between replays
