"""Properties of the GPU path that hold at any size: chunk-size invariance,
packing, state handoff, value-column separability, run-to-run determinism."""
import pytest
import torch

import workloads
from kda_testutil import (TOL_BF16, dev, gpu_or_skip, gpu_prefill, np64, oracle_on,
                          assert_parity, rel_fro)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def test_chunk_invariance_f32():
    """fp32: chunk 16, 32 and 64 agree to fp32 rounding (the chunked form is exact)."""
    kda()
    inp = workloads.recurrence_inputs([200, 77], H=2, d=64, dtype="f32", s0_std=0.3, seed=21)
    res = [gpu_prefill(inp, chunk=c) for c in (16, 32, 64)]
    for o, S in res[1:]:
        assert rel_fro(np64(o), np64(res[0][0])) < 1e-5
        assert rel_fro(np64(S), np64(res[0][1])) < 1e-5


def test_chunk_invariance_mfma_vs_vector():
    """bf16 d=128: the matrix-core kernel (chunk 64) and the vector kernel (chunk
    16, fp32 math on the same bf16 inputs) agree within the bf16 budget."""
    kda()
    inp = workloads.recurrence_inputs([500], H=4, d=128, dtype="bf16", g_mu=3.0, g_sigma=1.0,
                                      seed=22)
    o64, S64 = gpu_prefill(inp, chunk=64)
    o16, S16 = gpu_prefill(inp, chunk=16)
    e = max(rel_fro(np64(o64), np64(o16)), rel_fro(np64(S64), np64(S16)))
    print(f"mfma vs vector: {e:.2e}")
    assert e <= TOL_BF16


@pytest.mark.parametrize("d,dtype,ws", [(128, "bf16", "auto"), (128, "bf16", None),
                                         (32, "f32", None)])
def test_packing_is_exact(d, dtype, ws):
    """A packed call equals separate per-sequence calls, bit for bit."""
    kda()
    lens = [70, 3, 130]
    inp = workloads.recurrence_inputs(lens, H=8, d=d, dtype=dtype, s0_std=0.2, seed=23)
    o, S = gpu_prefill(inp, workspace=ws)
    cu = inp.cu_seqlens.tolist()
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        sub = workloads.RecurrenceInputs(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl],
                                         inp.beta[sl],
                                         torch.tensor([0, lens[n]], dtype=torch.int32),
                                         inp.S0[n:n + 1], dtype, inp.chunk)
        on, Sn = gpu_prefill(sub, workspace=ws)
        assert torch.equal(on, o[sl]) and torch.equal(Sn[0], S[n])


def test_split_and_fused_agree():
    """The two matrix-core paths compute the same chunked form: they agree far
    inside the bf16 budget on a multi-chunk, multi-head input."""
    kda()
    inp = workloads.recurrence_inputs([700, 300], H=8, d=128, dtype="bf16", g_mu=3.0,
                                      g_sigma=1.0, s0_std=0.3, seed=24)
    o1, S1 = gpu_prefill(inp, workspace="auto")
    o2, S2 = gpu_prefill(inp, workspace=None)
    e = max(rel_fro(np64(o1), np64(o2)), rel_fro(np64(S1), np64(S2)))
    print(f"split vs fused: {e:.2e}")
    assert e <= TOL_BF16 / 4


@pytest.mark.parametrize("workspace", ["auto", None])
def test_strong_decay_within_range(workspace):
    """Decay strong enough (alpha ~ 0.3 per token and channel) that a 64-token
    chunk's cumulative log decay reaches about -77 in some channels: the
    matrix-core paths reference the decay to the chunk's end, so their factor
    e^(b_t - b_C) then reaches ~e^77, near the fp32 limit (~e^88).  Both paths
    still match the oracle."""
    kda()
    inp = workloads.recurrence_inputs([256, 100], H=2, d=128, dtype="bf16", g_mu=-0.84,
                                      g_sigma=0.1, s0_std=0.3, seed=25)
    cu = [int(c) for c in inp.cu_seqlens]
    lows = [float(inp.g[t:min(t + 64, cu[n + 1])].sum(0).min())
            for n in range(len(cu) - 1) for t in range(cu[n], cu[n + 1], 64)]
    assert -88.0 < min(lows) < -70.0, min(lows)
    o, S = gpu_prefill(inp, workspace=workspace)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"strong decay ({'two-kernel' if workspace else 'fused'}), lowest chunk "
                  f"log decay {min(lows):.1f}")


def test_handoff_prefill_prefill():
    """prefill(T1) then prefill(T2) from its final state equals prefill(T1 + T2)."""
    kda()
    inp = workloads.recurrence_inputs([300], H=4, d=128, dtype="bf16", s0_std=0.1, seed=24)
    o, S = gpu_prefill(inp)
    T1 = 137
    a = workloads.RecurrenceInputs(inp.q[:T1], inp.k[:T1], inp.v[:T1], inp.g[:T1],
                                   inp.beta[:T1], torch.tensor([0, T1], dtype=torch.int32),
                                   inp.S0, "bf16", 64)
    oa, Sa = gpu_prefill(a)
    b = workloads.RecurrenceInputs(inp.q[T1:], inp.k[T1:], inp.v[T1:], inp.g[T1:],
                                   inp.beta[T1:],
                                   torch.tensor([0, 300 - T1], dtype=torch.int32), Sa.cpu(),
                                   "bf16", 64)
    ob, Sb = gpu_prefill(b)
    e = max(rel_fro(np64(torch.cat([oa, ob])), np64(o)), rel_fro(np64(Sb), np64(S)))
    print(f"handoff: {e:.2e}")
    assert e <= TOL_BF16


def test_value_column_separability():
    """Columns of o and S depend only on the same columns of v and S_0: changing
    v and S_0 in value columns 64..127 leaves columns 0..63 unchanged, bit for bit
    (the kernels slice the state by value columns)."""
    kda()
    inp = workloads.recurrence_inputs([150], H=2, d=128, dtype="bf16", s0_std=0.2, seed=25)
    o1, S1 = gpu_prefill(inp)
    v2 = inp.v.clone()
    v2[..., 64:] = -v2[..., 64:] * 3
    S02 = inp.S0.clone()
    S02[..., 64:] = 1.0
    inp2 = workloads.RecurrenceInputs(inp.q, inp.k, v2, inp.g, inp.beta, inp.cu_seqlens, S02,
                                      "bf16", 64)
    o2, S2 = gpu_prefill(inp2)
    assert torch.equal(o1[..., :64], o2[..., :64])
    assert torch.equal(S1[..., :64], S2[..., :64])


def test_determinism():
    """Two identical runs give identical bytes (no race on LDS)."""
    kda()
    inp = workloads.recurrence_inputs([257, 64], H=8, d=128, dtype="bf16", s0_std=0.1, seed=26)
    o1, S1 = gpu_prefill(inp)
    o2, S2 = gpu_prefill(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_graph_capture_replays():
    """The whole hot path (state init, two-kernel prefill, a decode step, a
    two-token decode) captured in one HIP graph and replayed several times, with
    eager work in between: every replay equals the eager run, bit for bit."""
    m = kda()
    inp = workloads.recurrence_inputs([200, 77], H=4, d=128, dtype="bf16", s0_std=0.3, seed=31)
    dec = workloads.recurrence_inputs([1, 1], H=4, d=128, dtype="bf16", seed=32)
    two = workloads.recurrence_inputs([2, 2], H=4, d=128, dtype="bf16", seed=33)
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    dq, dk, dv, dg, db = (dev(x) for x in (dec.q, dec.k, dec.v, dec.g, dec.beta))
    t2 = lambda x: dev(x.reshape((2, 2) + tuple(x.shape[1:])))
    tq, tk, tv, tg, tb = (t2(x) for x in (two.q, two.k, two.v, two.g, two.beta))
    cu, s0 = dev(inp.cu_seqlens), dev(inp.S0)
    state = torch.empty_like(s0)
    o, od, ot = torch.empty_like(q), torch.empty_like(dq), torch.empty_like(tv)
    ws = torch.empty(m.kda_prefill_workspace_bytes(2, 4, 128, 128, 64, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def run():
        m.kda_state_init(state, s0)
        m.kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=inp.cu_seqlens,
                              initial_state=state, final_state=state, o=o, workspace=ws)
        m.kda_decode_step(dq, dk, dv, dg, db, state, o=od)
        m.kda_decode_tokens(tq, tk, tv, tg, tb, state, o=ot)

    run()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, od, ot, state)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for _ in range(4):
        for x in (o, od, ot, state):
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip((o, od, ot, state), ref):
            assert torch.equal(x, y)


def test_two_streams_concurrent_prefills():
    """Two prefills enqueued on two streams at once, each through the binding's
    default workspace (one cached buffer per device and stream, so they do not
    share tiles): both match the oracle and equal the same calls made one after
    the other on the current stream, bit for bit."""
    m = kda()
    a = workloads.recurrence_inputs([700, 300], H=8, d=128, dtype="bf16", s0_std=0.2, seed=41)
    b = workloads.recurrence_inputs([900, 64, 257], H=8, d=128, dtype="bf16", s0_std=0.2,
                                    seed=42)
    ref_a = gpu_prefill(a)
    ref_b = gpu_prefill(b)
    args = []
    for inp in (a, b):
        args.append((dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                     dev(inp.cu_seqlens), inp.cu_seqlens, dev(inp.S0)))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [None, None]
    for rep in range(3):
        for i, st in enumerate((s1, s2)):
            q, k, v, g, beta, cu, cu_h, s0 = args[i]
            with torch.cuda.stream(st):
                outs[i] = m.kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu,
                                                cu_seqlens_host=cu_h, initial_state=s0,
                                                stream=st)
        torch.cuda.synchronize()
        for (o, S), (o_r, S_r) in zip(outs, (ref_a, ref_b)):
            assert torch.equal(o, o_r) and torch.equal(S, S_r), rep
    for inp, (o, S) in zip((a, b), outs):
        o_ref, S_ref = oracle_on(inp)
        assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                      "prefill on its own stream")
