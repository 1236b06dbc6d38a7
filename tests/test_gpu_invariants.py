"""Properties of the GPU path that hold at any size: chunk-size invariance,
packing, state handoff, value-column separability, run-to-run determinism."""
import pytest
import torch

import workloads
from kda_testutil import (TOL_BF16, TOL_F32, dev, gpu_or_skip, gpu_prefill, np64, oracle_on,
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


def chunk_log_decays(inp):
    """Lowest cumulative log decay over any chunk (per channel and head)."""
    cu = [int(c) for c in inp.cu_seqlens]
    return min(float(inp.g[t:min(t + inp.chunk, cu[n + 1])].sum(0).min())
               for n in range(len(cu) - 1) for t in range(cu[n], cu[n + 1], inp.chunk))


# (label, d, dtype, chunk, workspace): the two-kernel and fused matrix-core
# paths and the vector kernel (bf16 at chunk 32, fp32 at chunk 64)
DECAY_PATHS = [("split", 128, "bf16", 64, "auto"), ("fused", 128, "bf16", 64, None),
               ("vector_bf16", 128, "bf16", 32, None), ("vector_f32", 64, "f32", 64, None)]


@pytest.mark.parametrize("label,d,dtype,chunk,ws", DECAY_PATHS, ids=[p[0] for p in DECAY_PATHS])
@pytest.mark.parametrize("regime", ["moderate", "clamped", "extreme", "mixed"])
def test_decay_range(label, d, dtype, chunk, ws, regime):
    """Decays over the whole range, against the oracle by every measure:
      moderate: alpha ~ 0.3 per token on every channel, a chunk of 64 decaying by
                about e^-77 (the operands' reference sits at the chunk's end);
      clamped:  alpha ~ e^-1.5, about e^-100 per chunk of 64 (the reference is
                clamped, the factored products still hold);
      extreme:  16 channels of every head at alpha ~ e^-4.7, about e^-300 per
                chunk of 64, beside ordinary ones (the pairwise path);
      mixed:    the extreme channels only on tokens [128, 320), so that chunks
                on the pairwise path and factored ones alternate in a sequence
                and hand the state to each other."""
    kda()
    lens = [520, 100, 0, 64]
    base = dict(H=3, d=d, dtype=dtype, chunk=chunk, s0_std=0.3, seed=25 + d + chunk)
    if regime == "moderate":
        inp = workloads.recurrence_inputs(lens, g_mu=-0.84, g_sigma=0.1, **base)
    elif regime == "clamped":
        inp = workloads.recurrence_inputs(lens, g_mu=-1.2, g_sigma=0.1, **base)
    else:
        inp = workloads.recurrence_inputs(lens, g_mu=3.0, g_sigma=1.0, **base)
        tokens = None if regime == "extreme" else (128, 320)
        inp = workloads.with_strong_decay(inp, range(0, d, d // 16), tokens=tokens, seed=26)
    low = chunk_log_decays(inp)
    o, S = gpu_prefill(inp, workspace=ws)
    o_ref, S_ref = oracle_on(inp)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, tol,
                  f"decay {regime} ({label}), lowest chunk log decay {low:.1f}")


@pytest.mark.parametrize("ws", ["auto", None], ids=["split", "fused"])
def test_decay_range_gate_proj(ws):
    """The fused gate prologue with f ~ N(0, 1) and a rate exp(a_log) = 8 on every
    head: log alpha = -8 softplus(f), about -6.5 per token on average, chunks of
    64 decaying by e^-300 to e^-600 on every channel."""
    m = kda()
    import math
    import oracle
    lens, H, d = [300, 64, 130], 4, 128
    inp = workloads.recurrence_inputs(lens, H=H, d=d, dtype="bf16", chunk=64, s0_std=0.3,
                                      seed=27)
    pr = workloads.gate_projections(inp.T, H, d, dtype="bf16", g_mu=0.0, g_sigma=1.0, seed=28)
    a_log = torch.full((H,), math.log(8.0))
    g, beta = oracle.gate_prologue(np64(pr.f), np64(a_log), np64(pr.b))
    ref = workloads.RecurrenceInputs(inp.q, inp.k, inp.v, torch.from_numpy(g),
                                     torch.from_numpy(beta), inp.cu_seqlens, inp.S0, "bf16", 64)
    low = chunk_log_decays(ref)
    o, S = m.kda_prefill_chunked(dev(inp.q), dev(inp.k), dev(inp.v), dev(pr.f), dev(pr.b),
                                 cu_seqlens=dev(inp.cu_seqlens), cu_seqlens_host=inp.cu_seqlens,
                                 initial_state=dev(inp.S0), workspace=ws, a_log=dev(a_log))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(ref)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"gate prologue at rate 8, lowest chunk log decay {low:.1f}")


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
