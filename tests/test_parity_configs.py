"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times.  Where the oracle cannot afford every head, it runs on a sample
of heads (the recurrence is independent per head) and those heads are compared
in full: every token's output row and every sequence's final state, per
sequence, per (sequence, head) and per row (kda_testutil.assert_parity).

Tolerances: max relative Frobenius error of outputs and final states <= 1e-4 for
fp32 inputs, <= 2e-2 for bf16 inputs with fp32 state."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from kda_testutil import (TOL_BF16, TOL_F32, dev, gpu_or_skip, gpu_prefill, np64, oracle_on,
                          assert_parity, rel_fro)

pytestmark = pytest.mark.gpu


def kda():
    gpu_or_skip()
    import gated_delta_rule_99_amd as m
    m.load()
    return m


def test_config_tiny_f32():
    kda()
    inp = workloads.tiny_f32()
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_F32,
                  f"tiny f32")


def test_config_ling_prefill():
    """B=1, H=64, T=8192, d=128, chunk 64, bf16; every head checked."""
    kda()
    inp = workloads.ling_prefill()
    o, S = gpu_prefill(inp)
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(S), S_ref, inp.cu_seqlens, TOL_BF16, "ling prefill")


def test_config_decode_batch():
    """B=256 x H=64 decode step from random N(0, 0.02) states; every state checked."""
    m = kda()
    inp = workloads.decode_batch()
    state = dev(inp.S0)
    o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_on(inp)
    assert_parity(np64(o), o_ref, np64(state), S_ref, inp.cu_seqlens, TOL_BF16,
                  f"decode batch")


def test_config_decode_batch_bf16_state():
    """The same step on states stored in bf16: outputs against the oracle run from
    the stored values, every written state against the oracle's final state
    rounded to bf16 (one bf16 spacing, plus fp32 slack where a step cancels)."""
    m = kda()
    inp = workloads.decode_batch()
    S0 = torch.from_numpy(oracle.round_bf16(inp.S0.double().numpy())).float()
    state = dev(S0.to(torch.bfloat16))
    o = m.kda_decode_step(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state)
    torch.cuda.synchronize()
    ref = workloads.RecurrenceInputs(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, S0,
                                     "bf16", inp.chunk)
    o_ref, S_ref = oracle_on(ref)
    want = oracle.round_bf16(S_ref)
    got = state.float().cpu().double().numpy()
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    assert_parity(np64(o), o_ref, got, S_ref, inp.cu_seqlens, TOL_BF16,
                  "decode batch, bf16 state")
    exact = float(np.mean(got == want))
    print(f"state elements equal to the rounded oracle: {exact:.5f}")
    assert np.all(np.abs(got - want) <= spacing * (1 + 1e-9) + 1e-6)
    assert exact >= 0.999


# heads of the two long sequences checked against the oracle (every fourth);
# the two shorter sequences are checked on every head
PACKED_HEADS = tuple(range(0, 64, 4))


def oracle_seq(inp, n, heads):
    """Oracle on sequence n alone, on the given heads: (o [len, |heads|, dv],
    S [1, |heads|, dk, dv])."""
    a, b = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
    sub = workloads.RecurrenceInputs(inp.q[a:b], inp.k[a:b], inp.v[a:b], inp.g[a:b],
                                     inp.beta[a:b], torch.tensor([0, b - a], dtype=torch.int32),
                                     None if inp.S0 is None else inp.S0[n:n + 1], inp.dtype,
                                     inp.chunk)
    return oracle_on(sub, heads=heads)


def test_config_packed_long():
    """Sequences of 131072, 65536, 16384 and 1000 tokens, nonzero initial states.
    The two shorter sequences are checked on every head, the two long ones on
    16 heads (every fourth): every token's output row and the final state of
    each checked (sequence, head), by every measure of assert_parity."""
    kda()
    inp = workloads.packed_long()
    o, S = gpu_prefill(inp)
    cu = inp.cu_seqlens.tolist()
    for n in range(inp.n_seqs):
        heads = list(PACKED_HEADS) if cu[n + 1] - cu[n] > 20000 else list(range(inp.H))
        o_s = np64(o[cu[n]:cu[n + 1], heads])
        S_s = np64(S[n:n + 1, heads])
        o_ref, S_ref = oracle_seq(inp, n, heads)
        assert_parity(o_s, o_ref, S_s, S_ref, [0, cu[n + 1] - cu[n]], TOL_BF16,
                      f"packed long, sequence {n} ({cu[n + 1] - cu[n]} tokens, "
                      f"{len(heads)} heads)")
        # early outputs carry the initial state's influence: check them on their own
        assert_parity(o_s[:64], o_ref[:64], None, None, [0, 64], TOL_BF16,
                      f"packed long, sequence {n}, first 64 tokens")
        del o_s, o_ref


def test_ragged_batch_growing_windows():
    """Six sequences of different lengths (one empty, one shorter than a chunk)
    at H=64, nonzero initial states, two-kernel path with the minimum workspace:
    the windows start at 7 chunks for six running sequences and grow to 32 as
    the shorter ones end.  Every sequence's outputs and final state on every
    head, and the empty sequence's final state equal to its initial one."""
    m = kda()
    lens = [64 * 40, 64 * 3 + 5, 0, 64 * 70 + 1, 17, 64 * 33]
    inp = workloads.recurrence_inputs(lens, H=64, d=128, dtype="bf16", chunk=64, s0_std=0.05,
                                      seed=1010)
    need = m.kda_prefill_workspace_bytes(len(lens), 64, 128, 128, 64, torch.bfloat16)
    o, S = gpu_prefill(inp, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    o_s, S_s = np64(o), np64(S)
    assert torch.equal(S[2].cpu(), inp.S0[2])
    del o, S
    o_ref, S_ref = oracle_on(inp)
    assert_parity(o_s, o_ref, S_s, S_ref, inp.cu_seqlens, TOL_BF16,
                  f"ragged batch, growing windows")


def test_batch_with_long_windows():
    """24 sequences of 2048 tokens at H=64 through the binding's default
    workspace, which holds all 32 chunks of every sequence in one window; the
    same batch with the minimum workspace (windows of 1 chunk) gives the same
    result up to rounding.  Sixteen heads (every fourth) against the oracle."""
    m = kda()
    inp = workloads.recurrence_inputs([2048] * 24, H=64, d=128, dtype="bf16", chunk=64,
                                      s0_std=0.05, seed=1011)
    o, S = gpu_prefill(inp)
    need = m.kda_prefill_workspace_bytes(24, 64, 128, 128, 64, torch.bfloat16)
    o1, S1 = gpu_prefill(inp, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    heads = list(range(3, 64, 4))
    o_s, S_s = np64(o[:, heads]), np64(S[:, heads])
    assert rel_fro(np64(o1[:, heads]), o_s) <= 1e-2
    del o, S, o1, S1
    o_ref, S_ref = oracle_on(inp, heads=heads)
    assert_parity(o_s, o_ref, S_s, S_ref, inp.cu_seqlens, TOL_BF16,
                  f"batch of 24 x 2048, 32-chunk windows")


def run_mixer_gpu(m, mi):
    """Conv + L2 front end, chunked prefill, then recurrent decode steps, all
    through the C ABI.  Returns (o_prefill, o_decode, final_state)."""
    H, d, Tp = mi.H, mi.d, mi.t_prefill
    Cch = H * d
    w = {s: dev(getattr(mi, "w_" + s)) for s in "qkv"}
    x = {s: getattr(mi, "x_" + s) for s in "qkv"}
    tails = {s: torch.empty((1, 3, Cch), dtype=torch.bfloat16, device="cuda") for s in "qkv"}
    y = {}
    for s in "qkv":
        y[s] = m.kda_short_conv_prefill(dev(x[s][:Tp]), w[s], l2_head_dim=0 if s == "v" else d,
                                        l2_eps=1e-6, conv_tail_out=tails[s])
    g = dev(mi.g)
    beta = dev(mi.beta)
    o_pre, S = m.kda_prefill_chunked(y["q"].view(Tp, H, d), y["k"].view(Tp, H, d),
                                     y["v"].view(Tp, H, d), g[:Tp].contiguous(),
                                     beta[:Tp].contiguous(), chunk=mi.chunk)
    outs = []
    xd = {s: dev(x[s][Tp:]) for s in "qkv"}
    for t in range(mi.n_decode):
        yd = {}
        for s in "qkv":
            yd[s] = m.kda_short_conv_decode(xd[s][t:t + 1], w[s], tails[s],
                                            l2_head_dim=0 if s == "v" else d, l2_eps=1e-6)
        outs.append(m.kda_decode_step(yd["q"].view(1, H, d), yd["k"].view(1, H, d),
                                      yd["v"].view(1, H, d), g[Tp + t:Tp + t + 1],
                                      beta[Tp + t:Tp + t + 1], S))
    torch.cuda.synchronize()
    return o_pre, torch.cat(outs), S


def oracle_mixer(mi, heads):
    """Oracle: conv (fp64) over all prefill + decode tokens of the given heads'
    channels, L2 per head on q and k, one recurrence over every token."""
    d = mi.d
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    streams = {}
    for s in "qkv":
        xs = np64(getattr(mi, "x_" + s)[:, cols])
        ws = np64(getattr(mi, "w_" + s)[cols])
        ys, _ = oracle.short_conv(xs, ws)
        if s != "v":
            ys = oracle.l2norm_heads(ys, d, eps=1e-6)
        streams[s] = ys.reshape(ys.shape[0], len(heads), d)
    g = np64(mi.g[:, list(heads)])
    beta = np64(mi.beta[:, list(heads)])
    return oracle.recurrence(streams["q"], streams["k"], streams["v"], g, beta)


def test_config_mixer_handoff():
    """Conv + L2 + prefill of 32768 tokens, then 512 decode steps continuing from
    the prefill state and conv tails, against one 33280-token oracle run on
    every head: prefill outputs, decode outputs and the final state, each by
    every measure of assert_parity."""
    m = kda()
    mi = workloads.mixer()
    o_pre, o_dec, S = run_mixer_gpu(m, mi)
    o_ref, S_ref = oracle_mixer(mi, list(range(mi.H)))
    Tp = mi.t_prefill
    assert_parity(np64(o_pre), o_ref[:Tp], np64(S), S_ref, [0, Tp], TOL_BF16,
                  "mixer prefill outputs and final state")
    assert_parity(np64(o_dec), o_ref[Tp:], None, None, [0, mi.n_decode], TOL_BF16,
                  "mixer decode outputs")
